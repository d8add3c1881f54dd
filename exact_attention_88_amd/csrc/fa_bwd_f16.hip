// Backward dK/dV and dQ kernels for 16-bit inputs (fp16, bf16) with head dim
// 128 on gfx950: the tuned path.
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
//     transposed (ds_read_b64_tr_b16) is either stored once in an XOR-swizzled
//     unpadded layout that is conflict free for both read patterns (the
//     default variants: half the LDS stores and footprint), or twice, once
//     with the 16-byte row padding that makes 16-row ds_read_b128 reads
//     conflict free and once with the 64-byte padding that makes 4-row
//     transposed reads conflict free;
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

template <int ROWS, int NT, class T>
__device__ __forceinline__ void tile_load(u32x4* r, const T* __restrict__ base, int64_t ss,
                                          int row0, int nrows) {
  constexpr int PER = ROWS * 16 / NT;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * NT + (int)threadIdx.x;
    const int row = min(row0 + (c >> 4), nrows - 1);  // rows past the end are masked later
    r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ss + ((c & 15) << 3));
  }
}

template <int ROWS, int NT, int LS, class T>
__device__ __forceinline__ void tile_store(const u32x4* r, T* lds) {
  constexpr int PER = ROWS * 16 / NT;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * NT + (int)threadIdx.x;
    *reinterpret_cast<u32x4*>(lds + (c >> 4) * LS + ((c & 15) << 3)) = r[i];
  }
}

// Row-wise fragment (row-read layout): lane (c, g) gets row rbase + c, chunk kchunk + g.
template <class T>
__device__ __forceinline__ V8<T> frag_r(const T* lds, int rbase, int kchunk) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const V8<T>*>(lds + (rbase + (lane & 31)) * kLSR +
                                      (kchunk + (lane >> 5)) * 8);
}

// Transposed fragment (transposed-read layout); see frag_tr in fa_common.h.
template <class T>
__device__ __forceinline__ V8<T> frag_t(const T* lds, int rbase, int t, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 15;
  const int col = cbase + ((lane >> 4) & 1) * 16 + (j & 3) * 4;
  const int row = rbase + t * 16 + g * 4 + (j >> 2);
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const T* p0 = lds + row * kLST + col;
  s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
  s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 8 * kLST));
  V4<T> ah = __builtin_bit_cast(V4<T>, a), bh = __builtin_bit_cast(V4<T>, b);
  V8<T> r;
  r[0] = ah[0]; r[1] = ah[1]; r[2] = ah[2]; r[3] = ah[3];
  r[4] = bh[0]; r[5] = bh[1]; r[6] = bh[2]; r[7] = bh[3];
  return r;
}

// Single-copy swizzled layout: unpadded 256-byte rows in which the 16-byte
// chunk k of row r sits at chunk position k ^ swz(r).  swz(r) takes distinct
// values on any 16 consecutive rows (so 16-row ds_read_b128 row reads and
// full-row stores are conflict free) and, on 4 rows that start at a multiple
// of 4, spreads 4 neighbouring chunks over all 16 chunk positions (so 4-row
// transposed reads are conflict free).  One layout serves both read patterns.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int ROWS, int NT, class T>
__device__ __forceinline__ void tile_store_swz(const u32x4* r, T* lds) {
  constexpr int PER = ROWS * 16 / NT;
  static_assert(NT % 256 == 0, "every thread keeps its row residue mod 16");
  const int row0 = (int)threadIdx.x >> 4, off = row0 * kD + (((threadIdx.x & 15) ^ swz(row0)) << 3);
#pragma unroll
  for (int i = 0; i < PER; ++i) *reinterpret_cast<u32x4*>(lds + i * (NT / 16) * kD + off) = r[i];
}

// Row-wise fragment in the swizzled layout; rbase is a multiple of 16.
template <class T>
__device__ __forceinline__ V8<T> frag_r_swz(const T* lds, int rbase, int kchunk) {
  const int lane = threadIdx.x & 63, r = lane & 31;
  return *reinterpret_cast<const V8<T>*>(lds + (rbase + r) * kD +
                                      (((kchunk + (lane >> 5)) ^ swz(r)) << 3));
}

// Transposed fragment in the swizzled layout (same lanes as frag_t); rbase is
// a multiple of 16 and cbase of 8.
template <class T>
__device__ __forceinline__ V8<T> frag_t_swz(const T* lds, int rbase, int t, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 15;
  const int col = ((lane >> 4) & 1) * 16 + (j & 3) * 4;
  const int r = g * 4 + (j >> 2);
  const int ch = (cbase >> 3) + (col >> 3);
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const T* p0 = lds + (rbase + t * 16 + r) * kD + ((ch ^ swz(r)) << 3) + (col & 7);
  const T* p1 = lds + (rbase + t * 16 + r + 8) * kD + ((ch ^ swz(r + 8)) << 3) + (col & 7);
  s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
  s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1));
  V4<T> ah = __builtin_bit_cast(V4<T>, a), bh = __builtin_bit_cast(V4<T>, b);
  V8<T> x;
  x[0] = ah[0]; x[1] = ah[1]; x[2] = ah[2]; x[3] = ah[3];
  x[4] = bh[0]; x[5] = bh[1]; x[6] = bh[2]; x[7] = bh[3];
  return x;
}

// Accumulator registers t*8 .. t*8+7 rounded to T (round to nearest even).
template <class T>
__device__ __forceinline__ V8<T> cvt8(const f32x16& x, int t) {
  V8<T> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)x[t * 8 + e];
  return r;
}

template <class T>
__device__ __forceinline__ void store_row4x4(T* rowp, const f32x16* acc, float mul, int g) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      V4<T> v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (T)(acc[db][r4 * 4 + e] * mul);
      *reinterpret_cast<V4<T>*>(rowp + db * 32 + r4 * 8 + g * 4) = v;
    }
}

// ------------------------------------------------------------------- dQ
// SWZ: K and V are stored once each in the swizzled layout (K serves both its
// row-wise and its transposed reads) instead of K twice in the padded layouts.
template <class T, int BN, int NW, bool CAUSAL, bool SWZ>
__global__ __launch_bounds__(NW * 64, 2) void dq_f16_d128(BwdArgs a) {
  constexpr int BM = 32 * NW, NT = NW * 64, NKB = BN / 32;
  constexpr int TR = SWZ ? BN * kD : BN * kLSR, TT = SWZ ? 0 : BN * kLST;
  constexpr int BUF = 2 * TR + TT;  // K rows, V rows[, K transposed]
  __shared__ __attribute__((aligned(1024))) T smem[2 * BUF];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  const int L = xcd_logical_block();
  int qb = L % nqb;
  const int bh = L / nqb;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;
  const bool valid = qi < a.Sq;

  V8<T> qf[8], df[8];
  {
    const int qc = min(qi, a.Sq - 1);
    const T* qrow = (const T*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qc * a.q.ss;
    const T* drow =
        (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh + (int64_t)qc * a.dout.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const V8<T>*>(qrow + ks * 16 + g * 8);
      df[ks] = *reinterpret_cast<const V8<T>*>(drow + ks * 16 + g * 8);
    }
  }
  // Rows past the end, and rows with no visible key (LSE = -inf), get P = 0.
  const float lse_n = valid ? a.lse[(int64_t)bh * a.Sq + qi] : INFINITY;
  const float lse2 = lse_n == -INFINITY ? INFINITY : lse_n * kLog2e;
  const float dlt = valid ? a.delta[(int64_t)bh * a.Sq + qi] : 0.f;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): row data resident before the tile loop

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = zero16();
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  constexpr int PER = BN * 16 / NT;
  u32x4 kr[PER], vr[PER];
  tile_load<BN, NT>(kr, kbase, a.k.ss, 0, a.Sk);
  tile_load<BN, NT>(vr, vbase, a.v.ss, 0, a.Sk);
  auto store_tiles = [&](T* nb) {
    if constexpr (SWZ) {
      tile_store_swz<BN, NT>(kr, nb);
      tile_store_swz<BN, NT>(vr, nb + TR);
    } else {
      tile_store<BN, NT, kLSR>(kr, nb);
      tile_store<BN, NT, kLSR>(vr, nb + TR);
      tile_store<BN, NT, kLST>(kr, nb + 2 * TR);
    }
  };
  store_tiles(smem);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const T* Kr = smem + (t & 1) * BUF;
    const T* Vr = Kr + TR;
    const T* Kt = SWZ ? Kr : Kr + 2 * TR;
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) {
      tile_load<BN, NT>(kr, kbase, a.k.ss, k0 + BN, a.Sk);
      tile_load<BN, NT>(vr, vbase, a.v.ss, k0 + BN, a.Sk);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int ks0 = k0 + kb * 32;
      if (CAUSAL && ks0 > qw + a.coff + 31) continue;
      // Row-wise operands of S^T and dP^T first, then the transposed K operand
      // of dQ (one k-step at a time: with 8 waves a wave has 256 registers).
      V8<T> kf[8], vf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kf[ks] = SWZ ? frag_r_swz(Kr, kb * 32, ks * 2) : frag_r(Kr, kb * 32, ks * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        vf[ks] = SWZ ? frag_r_swz(Vr, kb * 32, ks * 2) : frag_r(Vr, kb * 32, ks * 2);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = Mfma<T>::mma(kf[ks], qf[ks], s);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dp = Mfma<T>::mma(vf[ks], df[ks], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(__builtin_fmaf(s[r], cs, -lse2));
      // Masks only on the diagonal block and the ragged key tail.
      if ((ks0 + 32 > a.Sk) || (CAUSAL && ks0 + 31 > qw + a.coff)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ks0 + crow(r, g);
          if (key >= a.Sk || (CAUSAL && key > qi + a.coff)) s[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - dlt);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        V8<T> kt[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          kt[db] = SWZ ? frag_t_swz(Kt, kb * 32, tt, db * 32) : frag_t(Kt, kb * 32, tt, db * 32);
        const V8<T> sf = cvt8<T>(s, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dq[db] = Mfma<T>::mma(kt[db], sf, dq[db]);
      }
    }
    if (more) store_tiles(smem + ((t + 1) & 1) * BUF);
  }

  if (valid) {
    T* row = (T*)a.dq.p + b * a.dq.sb + h * a.dq.sh + (int64_t)qi * a.dq.ss;
    store_row4x4(row, dq, a.scale, g);
  }
}

// ------------------------------------------------------------------- dK / dV
// SWZ: Q and dO are stored once each in the swizzled layout instead of twice
// in the padded layouts.
template <class T, int BM, int NW, bool CAUSAL, bool SWZ>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_f16_d128(BwdArgs a) {
  constexpr int BN = 32 * NW, NT = NW * 64, NQB = BM / 32;
  constexpr int TR = SWZ ? BM * kD : BM * kLSR, TT = SWZ ? 0 : BM * kLST;
  constexpr int BUF = 2 * TR + 2 * TT;  // Q rows, dO rows[, Q transposed, dO transposed]
  __shared__ __attribute__((aligned(1024))) T smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float lsd[2][2][BM];  // [buffer][LSE*log2e, delta][row]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nkb = (a.Sk + BN - 1) / BN;
  const int L = xcd_logical_block();
  const int kb = L % nkb;  // causal: lowest key blocks (most work) first
  const int bh = L / nkb;
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* dobase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  const float* lse = a.lse + (int64_t)bh * a.Sq;
  const float* dl = a.delta + (int64_t)bh * a.Sq;
  const int k0 = kb * BN, kw = k0 + w * 32, kj = kw + c;

  V8<T> kf[8], vf[8];
  {
    const int kc = min(kj, a.Sk - 1);
    const T* krow = (const T*)a.k.p + b * a.k.sb + h * a.k.sh + (int64_t)kc * a.k.ss;
    const T* vrow = (const T*)a.v.p + b * a.v.sb + h * a.v.sh + (int64_t)kc * a.v.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = *reinterpret_cast<const V8<T>*>(krow + ks * 16 + g * 8);
      vf[ks] = *reinterpret_cast<const V8<T>*>(vrow + ks * 16 + g * 8);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dk[i] = zero16(); dv[i] = zero16(); }
  const float cs = a.scale_log2;
  const bool key_tail = k0 + BN > a.Sk;

  const int qstart = CAUSAL ? (max(0, k0 - a.coff) / BM) * BM : 0;
  const int ntiles = a.Sq > qstart ? (a.Sq - qstart + BM - 1) / BM : 0;
  constexpr int PER = BM * 16 / NT;
  u32x4 qr[PER], dr[PER];
  // LSE and delta of the staged rows are loaded raw, unconditionally (the row
  // index clamped in bounds), and only converted when they are stored: a
  // select on a loaded value at the load site would make the wave wait for
  // that load, and with it for every tile load issued before it.
  float lsr = 0.f, dlr = 0.f;
  bool lrow = false;
  auto load_rows = [&](int q0) {
    tile_load<BM, NT>(qr, qbase, a.q.ss, q0, a.Sq);
    tile_load<BM, NT>(dr, dobase, a.dout.ss, q0, a.Sq);
    const int i = q0 + ((int)threadIdx.x & (BM - 1));
    lrow = i < a.Sq;
    lsr = lse[min(i, a.Sq - 1)];
    dlr = dl[min(i, a.Sq - 1)];
  };
  auto store_rows = [&](int buf) {
    T* base = smem + buf * BUF;
    if constexpr (SWZ) {
      tile_store_swz<BM, NT>(qr, base);
      tile_store_swz<BM, NT>(dr, base + TR);
    } else {
      tile_store<BM, NT, kLSR>(qr, base);
      tile_store<BM, NT, kLSR>(dr, base + TR);
      tile_store<BM, NT, kLST>(qr, base + 2 * TR);
      tile_store<BM, NT, kLST>(dr, base + 2 * TR + TT);
    }
    if ((int)threadIdx.x < BM) {
      // Rows past the end, and rows with no visible key (LSE = -inf), get P = 0.
      lsd[buf][0][threadIdx.x] = (!lrow || lsr == -INFINITY) ? INFINITY : lsr * kLog2e;
      lsd[buf][1][threadIdx.x] = lrow ? dlr : 0.f;
    }
  };
  if (ntiles > 0) {
    load_rows(qstart);
    store_rows(0);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int q0 = qstart + t * BM;
    const int buf = t & 1;
    const T* Qr = smem + buf * BUF;
    const T* Dr = Qr + TR;
    const T* Qt = SWZ ? Qr : Qr + 2 * TR;
    const T* Dt = SWZ ? Dr : Qt + TT;
    const float* Ls = lsd[buf][0];
    const float* Dl = lsd[buf][1];
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) load_rows(q0 + BM);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qs = q0 + qb * 32;
      if (CAUSAL && qs + a.coff + 31 < kw) continue;  // every query of the block precedes every key
      // Row-wise operands first (S and dP do not depend on each other), then the
      // transposed operands of dV and dK, so LDS latency overlaps the MFMAs.
      V8<T> qf[8], of[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qf[ks] = SWZ ? frag_r_swz(Qr, qb * 32, ks * 2) : frag_r(Qr, qb * 32, ks * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        of[ks] = SWZ ? frag_r_swz(Dr, qb * 32, ks * 2) : frag_r(Dr, qb * 32, ks * 2);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = Mfma<T>::mma(qf[ks], kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dp = Mfma<T>::mma(of[ks], vf[ks], dp);
      V8<T> dt[2][4], qt[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dt[tt][db] = SWZ ? frag_t_swz(Dt, qb * 32, tt, db * 32) : frag_t(Dt, qb * 32, tt, db * 32);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          qt[tt][db] = SWZ ? frag_t_swz(Qt, qb * 32, tt, db * 32) : frag_t(Qt, qb * 32, tt, db * 32);
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
      if (key_tail || (CAUSAL && qs + a.coff < kw + 31)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kj >= a.Sk || (CAUSAL && kj > qs + a.coff + crow(r, g))) p[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dr = r % 4 == 0 ? d4[r / 4].x : r % 4 == 1 ? d4[r / 4].y : r % 4 == 2 ? d4[r / 4].z : d4[r / 4].w;
        ds[r] = p[r] * (dp[r] - dr);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const V8<T> pf = cvt8<T>(p, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dv[db] = Mfma<T>::mma(dt[tt][db], pf, dv[db]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const V8<T> sf = cvt8<T>(ds, tt);
#pragma unroll
        for (int db = 0; db < 4; ++db) dk[db] = Mfma<T>::mma(qt[tt][db], sf, dk[db]);
      }
    }
    if (more) store_rows(buf ^ 1);
  }

  if (kj < a.Sk) {
    T* dkrow = (T*)a.dk.p + b * a.dk.sb + h * a.dk.sh + (int64_t)kj * a.dk.ss;
    T* dvrow = (T*)a.dv.p + b * a.dv.sb + h * a.dv.sh + (int64_t)kj * a.dv.ss;
    store_row4x4(dkrow, dk, a.scale, g);
    store_row4x4(dvrow, dv, 1.f, g);
  }
}

template <class T, int BN, int NW, bool CAUSAL, bool SWZ>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  constexpr int BM = 32 * NW;
  const int64_t grid = (((int64_t)a.Sq + BM - 1) / BM) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dq_f16_d128<T, BN, NW, CAUSAL, SWZ>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, s);
}

template <class T, int BM, int NW, bool CAUSAL, bool SWZ>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
  constexpr int BN = 32 * NW;
  const int64_t grid = (((int64_t)a.Sk + BN - 1) / BN) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dkdv_f16_d128<T, BM, NW, CAUSAL, SWZ>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, s);
}

}  // namespace

// dQ variants: 0 = (BN 64, 8 waves), 1 = (BN 64, 4 waves), 2 = (BN 32, 8 waves);
// 3, 4 = (BN 32, 64; 8 waves) with swizzled single-copy K and V.  (With
// 128-key tiles the staging registers push the non-causal kernel into spills.)
int dq_fast_variants() { return 5; }
TileCfg dq_fast_cfg(int v) {
  const int bn = v == 2 || v == 3 ? 32 : 64, nw = v == 1 ? 4 : 8;
  const int row_halfs = v >= 3 ? 2 * kD : 2 * kLSR + kLST;
  return TileCfg{32 * nw, bn, nw, 2 * bn * row_halfs * 2};
}
template <class T>
hipError_t launch_dq_variant(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dq_t<T, 64, 8, true, false>(a, s) : launch_dq_t<T, 64, 8, false, false>(a, s);
    case 1: return causal ? launch_dq_t<T, 64, 4, true, false>(a, s) : launch_dq_t<T, 64, 4, false, false>(a, s);
    case 2: return causal ? launch_dq_t<T, 32, 8, true, false>(a, s) : launch_dq_t<T, 32, 8, false, false>(a, s);
    case 3: return causal ? launch_dq_t<T, 32, 8, true, true>(a, s) : launch_dq_t<T, 32, 8, false, true>(a, s);
    case 4: return causal ? launch_dq_t<T, 64, 8, true, true>(a, s) : launch_dq_t<T, 64, 8, false, true>(a, s);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_dq_fast(const BwdArgs& a, int v, int dtype, int causal, hipStream_t s) {
  if (dtype == 2) return launch_dq_variant<bf16_t>(a, v, causal, s);
  return launch_dq_variant<half_t>(a, v, causal, s);
}

// dK/dV variants: 0 = (BM 64, 4 waves), 1 = (BM 32, 4 waves), 2 = (BM 64,
// 4 waves, swizzled single-copy Q and dO), 3 = (BM 128, 4 waves, swizzled).  (With 8 waves, two per SIMD, the
// 32 keys' K, V, dK and dV no longer fit the 256 registers a wave then gets,
// and the compiler spills.)
int dkdv_fast_variants() { return 4; }
TileCfg dkdv_fast_cfg(int v) {
  const int bm = v == 1 ? 32 : v == 3 ? 128 : 64, nw = 4;
  const int row_halfs = v >= 2 ? 2 * kD : 2 * kLSR + 2 * kLST;
  return TileCfg{bm, 32 * nw, nw, 2 * bm * row_halfs * 2 + 2 * 2 * bm * 4};
}
template <class T>
hipError_t launch_dkdv_variant(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dkdv_t<T, 64, 4, true, false>(a, s) : launch_dkdv_t<T, 64, 4, false, false>(a, s);
    case 1: return causal ? launch_dkdv_t<T, 32, 4, true, false>(a, s) : launch_dkdv_t<T, 32, 4, false, false>(a, s);
    case 2: return causal ? launch_dkdv_t<T, 64, 4, true, true>(a, s) : launch_dkdv_t<T, 64, 4, false, true>(a, s);
    case 3: return causal ? launch_dkdv_t<T, 128, 4, true, true>(a, s) : launch_dkdv_t<T, 128, 4, false, true>(a, s);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_dkdv_fast(const BwdArgs& a, int v, int dtype, int causal, hipStream_t s) {
  if (dtype == 2) return launch_dkdv_variant<bf16_t>(a, v, causal, s);
  return launch_dkdv_variant<half_t>(a, v, causal, s);
}

}  // namespace fa
