// Backward dK/dV and dQ kernels for fp16 with head dim 128 on gfx950: the
// tuned path.
//
// Same method as the generic backward kernels ("Triton FlashAttention": the
// FlashAttention-2 split into a dK/dV kernel and a dQ kernel with no atomics,
// probabilities rebuilt from the saved log-sum-exp; "FlashAttention-2 from
// PyTorch to Triton", the backward outline), laid out for CDNA4 like the tuned
// forward kernel:
//   * the streamed tiles are double-buffered in LDS through registers (the
//     global loads of tile t+1 are issued before tile t is computed), one
//     barrier per tile;
//   * a tile read both row-wise (as an untransposed MFMA operand) and
//     transposed (ds_read_b64_tr_b16) is stored twice, once with the 16-byte
//     row padding that makes 16-row ds_read_b128 reads conflict free and once
//     with the 64-byte padding that makes 4-row transposed reads conflict
//     free, so every fragment address is a base plus an immediate;
//   * all blocks of one (batch, head) are renumbered onto one XCD.
// dQ kernel: one workgroup per 32*waves query rows; Q, dO, LSE and delta of
// the wave's 32 rows live in registers, K and V stream (K in both layouts).
// dK/dV kernel: one workgroup per 32*waves keys; K and V of the wave's 32 keys
// live in registers, Q and dO stream in both layouts with LSE and delta.
#include "fa_args.h"
#include "fa_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kLSR = kD + 8;   // row-read layout stride (halfs): 272 bytes
constexpr int kLST = kD + 32;  // transposed-read layout stride (halfs): 320 bytes

__device__ __forceinline__ int xcd_logical_block() {
  const int n = gridDim.x, id = blockIdx.x;
  if (n % 8 != 0) return id;
  return (id % 8) * (n / 8) + id / 8;
}

template <int ROWS, int NT>
__device__ __forceinline__ void tile_load(u32x4* r, const half_t* __restrict__ base, int64_t ss,
                                          int row0, int nrows) {
  constexpr int PER = ROWS * 16 / NT;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * NT + (int)threadIdx.x;
    const int row = min(row0 + (c >> 4), nrows - 1);  // rows past the end are masked later
    r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ss + ((c & 15) << 3));
  }
}

template <int ROWS, int NT, int LS>
__device__ __forceinline__ void tile_store(const u32x4* r, half_t* lds) {
  constexpr int PER = ROWS * 16 / NT;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * NT + (int)threadIdx.x;
    *reinterpret_cast<u32x4*>(lds + (c >> 4) * LS + ((c & 15) << 3)) = r[i];
  }
}

// Row-wise fragment (row-read layout): lane (c, g) gets row rbase + c, chunk kchunk + g.
__device__ __forceinline__ h8 frag_r(const half_t* lds, int rbase, int kchunk) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const h8*>(lds + (rbase + (lane & 31)) * kLSR +
                                      (kchunk + (lane >> 5)) * 8);
}

// Transposed fragment (transposed-read layout); see frag_tr in fa_common.h.
__device__ __forceinline__ h8 frag_t(const half_t* lds, int rbase, int t, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 15;
  const int col = cbase + ((lane >> 4) & 1) * 16 + (j & 3) * 4;
  const int row = rbase + t * 16 + g * 4 + (j >> 2);
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const half_t* p0 = lds + row * kLST + col;
  s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
  s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 8 * kLST));
  h4 ah = __builtin_bit_cast(h4, a), bh = __builtin_bit_cast(h4, b);
  h8 r;
  r[0] = ah[0]; r[1] = ah[1]; r[2] = ah[2]; r[3] = ah[3];
  r[4] = bh[0]; r[5] = bh[1]; r[6] = bh[2]; r[7] = bh[3];
  return r;
}

__device__ __forceinline__ f32x16 mma(h8 a, h8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 cvt8(const f32x16& x, int t) {
  h8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (half_t)x[t * 8 + e];
  return r;
}

__device__ __forceinline__ void store_row4x4(half_t* rowp, const f32x16* acc, float mul, int g) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      h4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (half_t)(acc[db][r4 * 4 + e] * mul);
      *reinterpret_cast<h4*>(rowp + db * 32 + r4 * 8 + g * 4) = v;
    }
}

// ------------------------------------------------------------------- dQ
template <int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void dq_f16_d128(BwdArgs a) {
  constexpr int BM = 32 * NW, NT = NW * 64, NKB = BN / 32;
  constexpr int TR = BN * kLSR, TT = BN * kLST;
  constexpr int BUF = 2 * TR + TT;  // K rows, V rows, K transposed
  __shared__ __attribute__((aligned(1024))) half_t smem[2 * BUF];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  const int L = xcd_logical_block();
  int qb = L % nqb;
  const int bh = L / nqb;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const half_t* kbase = (const half_t*)a.k.p + b * a.k.sb + h * a.k.sh;
  const half_t* vbase = (const half_t*)a.v.p + b * a.v.sb + h * a.v.sh;
  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;
  const bool valid = qi < a.Sq;

  h8 qf[8], df[8];
  {
    const int qc = min(qi, a.Sq - 1);
    const half_t* qrow = (const half_t*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qc * a.q.ss;
    const half_t* drow =
        (const half_t*)a.dout.p + b * a.dout.sb + h * a.dout.sh + (int64_t)qc * a.dout.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const h8*>(qrow + ks * 16 + g * 8);
      df[ks] = *reinterpret_cast<const h8*>(drow + ks * 16 + g * 8);
    }
  }
  const float lse2 = valid ? a.lse[(int64_t)bh * a.Sq + qi] * kLog2e : INFINITY;
  const float dlt = valid ? a.delta[(int64_t)bh * a.Sq + qi] : 0.f;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): row data resident before the tile loop

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = zero16();
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? min(a.Sk, q0 + BM) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  constexpr int PER = BN * 16 / NT;
  u32x4 kr[PER], vr[PER];
  tile_load<BN, NT>(kr, kbase, a.k.ss, 0, a.Sk);
  tile_load<BN, NT>(vr, vbase, a.v.ss, 0, a.Sk);
  tile_store<BN, NT, kLSR>(kr, smem);
  tile_store<BN, NT, kLSR>(vr, smem + TR);
  tile_store<BN, NT, kLST>(kr, smem + 2 * TR);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const half_t* Kr = smem + (t & 1) * BUF;
    const half_t* Vr = Kr + TR;
    const half_t* Kt = Kr + 2 * TR;
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) {
      tile_load<BN, NT>(kr, kbase, a.k.ss, k0 + BN, a.Sk);
      tile_load<BN, NT>(vr, vbase, a.v.ss, k0 + BN, a.Sk);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int ks0 = k0 + kb * 32;
      if (CAUSAL && ks0 > qw + 31) continue;
      // Row-wise operands of S^T and dP^T first, then the transposed K operand
      // of dQ (one k-step at a time: with 8 waves a wave has 256 registers).
      h8 kf[8], vf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = frag_r(Kr, kb * 32, ks * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) vf[ks] = frag_r(Vr, kb * 32, ks * 2);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = mma(kf[ks], qf[ks], s);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dp = mma(vf[ks], df[ks], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(__builtin_fmaf(s[r], cs, -lse2));
      // Masks only on the diagonal block and the ragged key tail.
      if ((ks0 + 32 > a.Sk) || (CAUSAL && ks0 + 31 > qw)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ks0 + crow(r, g);
          if (key >= a.Sk || (CAUSAL && key > qi)) s[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - dlt);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        h8 kt[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) kt[db] = frag_t(Kt, kb * 32, tt, db * 32);
        const h8 sf = cvt8(s, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dq[db] = mma(kt[db], sf, dq[db]);
      }
    }
    if (more) {
      half_t* nb = smem + ((t + 1) & 1) * BUF;
      tile_store<BN, NT, kLSR>(kr, nb);
      tile_store<BN, NT, kLSR>(vr, nb + TR);
      tile_store<BN, NT, kLST>(kr, nb + 2 * TR);
    }
  }

  if (valid) {
    half_t* row = (half_t*)a.dq.p + b * a.dq.sb + h * a.dq.sh + (int64_t)qi * a.dq.ss;
    store_row4x4(row, dq, a.scale, g);
  }
}

// ------------------------------------------------------------------- dK / dV
template <int BM, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_f16_d128(BwdArgs a) {
  constexpr int BN = 32 * NW, NT = NW * 64, NQB = BM / 32;
  constexpr int TR = BM * kLSR, TT = BM * kLST;
  constexpr int BUF = 2 * TR + 2 * TT;  // Q rows, dO rows, Q transposed, dO transposed
  __shared__ __attribute__((aligned(1024))) half_t smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float lsd[2][2][BM];  // [buffer][LSE*log2e, delta][row]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nkb = (a.Sk + BN - 1) / BN;
  const int L = xcd_logical_block();
  const int kb = L % nkb;  // causal: lowest key blocks (most work) first
  const int bh = L / nkb;
  const int b = bh / a.H, h = bh % a.H;
  const half_t* qbase = (const half_t*)a.q.p + b * a.q.sb + h * a.q.sh;
  const half_t* dobase = (const half_t*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  const float* lse = a.lse + (int64_t)bh * a.Sq;
  const float* dl = a.delta + (int64_t)bh * a.Sq;
  const int k0 = kb * BN, kw = k0 + w * 32, kj = kw + c;

  h8 kf[8], vf[8];
  {
    const int kc = min(kj, a.Sk - 1);
    const half_t* krow = (const half_t*)a.k.p + b * a.k.sb + h * a.k.sh + (int64_t)kc * a.k.ss;
    const half_t* vrow = (const half_t*)a.v.p + b * a.v.sb + h * a.v.sh + (int64_t)kc * a.v.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = *reinterpret_cast<const h8*>(krow + ks * 16 + g * 8);
      vf[ks] = *reinterpret_cast<const h8*>(vrow + ks * 16 + g * 8);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dk[i] = zero16(); dv[i] = zero16(); }
  const float cs = a.scale_log2;
  const bool key_tail = k0 + BN > a.Sk;

  const int qstart = CAUSAL ? (k0 / BM) * BM : 0;
  const int ntiles = a.Sq > qstart ? (a.Sq - qstart + BM - 1) / BM : 0;
  constexpr int PER = BM * 16 / NT;
  u32x4 qr[PER], dr[PER];
  float lsr = 0.f, dlr = 0.f;
  auto load_rows = [&](int q0) {
    tile_load<BM, NT>(qr, qbase, a.q.ss, q0, a.Sq);
    tile_load<BM, NT>(dr, dobase, a.dout.ss, q0, a.Sq);
    if ((int)threadIdx.x < BM) {
      const int i = q0 + (int)threadIdx.x;
      lsr = i < a.Sq ? lse[i] * kLog2e : INFINITY;
      dlr = i < a.Sq ? dl[i] : 0.f;
    }
  };
  auto store_rows = [&](int buf) {
    half_t* base = smem + buf * BUF;
    tile_store<BM, NT, kLSR>(qr, base);
    tile_store<BM, NT, kLSR>(dr, base + TR);
    tile_store<BM, NT, kLST>(qr, base + 2 * TR);
    tile_store<BM, NT, kLST>(dr, base + 2 * TR + TT);
    if ((int)threadIdx.x < BM) {
      lsd[buf][0][threadIdx.x] = lsr;
      lsd[buf][1][threadIdx.x] = dlr;
    }
  };
  if (ntiles > 0) {
    load_rows(qstart);
    store_rows(0);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int q0 = qstart + t * BM;
    const int buf = t & 1;
    const half_t* Qr = smem + buf * BUF;
    const half_t* Dr = Qr + TR;
    const half_t* Qt = Qr + 2 * TR;
    const half_t* Dt = Qt + TT;
    const float* Ls = lsd[buf][0];
    const float* Dl = lsd[buf][1];
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) load_rows(q0 + BM);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qs = q0 + qb * 32;
      if (CAUSAL && qs + 31 < kw) continue;  // every query of the block precedes every key
      // Row-wise operands first (S and dP do not depend on each other), then the
      // transposed operands of dV and dK, so LDS latency overlaps the MFMAs.
      h8 qf[8], of[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = frag_r(Qr, qb * 32, ks * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) of[ks] = frag_r(Dr, qb * 32, ks * 2);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = mma(qf[ks], kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dp = mma(of[ks], vf[ks], dp);
      h8 dt[2][4], qt[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db) dt[tt][db] = frag_t(Dt, qb * 32, tt, db * 32);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db) qt[tt][db] = frag_t(Qt, qb * 32, tt, db * 32);
      // Per-row LSE and delta for the accumulator rows crow(r, g): 4 runs of 4.
      float4 l4[4], d4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l4[i] = *reinterpret_cast<const float4*>(Ls + qb * 32 + i * 8 + g * 4);
        d4[i] = *reinterpret_cast<const float4*>(Dl + qb * 32 + i * 8 + g * 4);
      }
      f32x16 p, ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float lr = r % 4 == 0 ? l4[r / 4].x : r % 4 == 1 ? l4[r / 4].y : r % 4 == 2 ? l4[r / 4].z : l4[r / 4].w;
        p[r] = fast_exp2(__builtin_fmaf(s[r], cs, -lr));
      }
      // Masks only on the diagonal block and the ragged key tail.
      if (key_tail || (CAUSAL && qs < kw + 31)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kj >= a.Sk || (CAUSAL && kj > qs + crow(r, g))) p[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dr = r % 4 == 0 ? d4[r / 4].x : r % 4 == 1 ? d4[r / 4].y : r % 4 == 2 ? d4[r / 4].z : d4[r / 4].w;
        ds[r] = p[r] * (dp[r] - dr);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const h8 pf = cvt8(p, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dv[db] = mma(dt[tt][db], pf, dv[db]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const h8 sf = cvt8(ds, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dk[db] = mma(qt[tt][db], sf, dk[db]);
      }
    }
    if (more) store_rows(buf ^ 1);
  }

  if (kj < a.Sk) {
    half_t* dkrow = (half_t*)a.dk.p + b * a.dk.sb + h * a.dk.sh + (int64_t)kj * a.dk.ss;
    half_t* dvrow = (half_t*)a.dv.p + b * a.dv.sb + h * a.dv.sh + (int64_t)kj * a.dv.ss;
    store_row4x4(dkrow, dk, a.scale, g);
    store_row4x4(dvrow, dv, 1.f, g);
  }
}

template <int BN, int NW, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  constexpr int BM = 32 * NW;
  const int64_t grid = (((int64_t)a.Sq + BM - 1) / BM) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dq_f16_d128<BN, NW, CAUSAL>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, s);
}

template <int BM, int NW, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
  constexpr int BN = 32 * NW;
  const int64_t grid = (((int64_t)a.Sk + BN - 1) / BN) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dkdv_f16_d128<BM, NW, CAUSAL>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, s);
}

}  // namespace

// dQ variants: 0 = (BN 64, 8 waves), 1 = (BN 64, 4 waves), 2 = (BN 32, 8 waves).
int dq_fast_variants() { return 3; }
TileCfg dq_fast_cfg(int v) {
  const int bn = v == 2 ? 32 : 64, nw = v == 1 ? 4 : 8;
  return TileCfg{32 * nw, bn, nw, 2 * bn * (2 * kLSR + kLST) * 2};
}
hipError_t launch_dq_fast(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dq_t<64, 8, true>(a, s) : launch_dq_t<64, 8, false>(a, s);
    case 1: return causal ? launch_dq_t<64, 4, true>(a, s) : launch_dq_t<64, 4, false>(a, s);
    case 2: return causal ? launch_dq_t<32, 8, true>(a, s) : launch_dq_t<32, 8, false>(a, s);
  }
  return hipErrorInvalidValue;
}

// dK/dV variants: 0 = (BM 64, 4 waves), 1 = (BM 32, 4 waves).  (With 8 waves,
// two per SIMD, the 32 keys' K, V, dK and dV no longer fit the 256 registers
// a wave then gets, and the compiler spills.)
int dkdv_fast_variants() { return 2; }
TileCfg dkdv_fast_cfg(int v) {
  const int bm = v == 1 ? 32 : 64, nw = 4;
  return TileCfg{bm, 32 * nw, nw, 2 * bm * (2 * kLSR + 2 * kLST) * 2 + 2 * 2 * bm * 4};
}
hipError_t launch_dkdv_fast(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dkdv_t<64, 4, true>(a, s) : launch_dkdv_t<64, 4, false>(a, s);
    case 1: return causal ? launch_dkdv_t<32, 4, true>(a, s) : launch_dkdv_t<32, 4, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
