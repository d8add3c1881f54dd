// Backward dK/dV and dQ kernels for 16-bit inputs (fp16, bf16) with head dim
// 128 (and, for the pipelined dK/dV and buffer-load dQ kernels, 64) on
// gfx950: the tuned path.
//
// Same method as the generic backward kernels ("Triton FlashAttention",
// opening summary: key-side and query-side gradients from two kernels, no
// atomics, probabilities recomputed from the saved log-sum-exp;
// "FlashAttention-2 from PyTorch to Triton", backward outline), laid out for
// CDNA4 like the tuned forward kernel:
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
#include <type_traits>

#include "fa_args.h"
#include "fa_common.h"
#include "fa_lds.h"

namespace fa {

namespace {

using namespace swzl;

constexpr int kLSR = kD + 8;   // row-read layout stride (halfs): 272 bytes
constexpr int kLST = kD + 32;  // transposed-read layout stride (halfs): 320 bytes

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

// Accumulator registers t*8 .. t*8+7 rounded to T (round to nearest even).
template <class T>
__device__ __forceinline__ V8<T> cvt8(const f32x16& x, int t) {
  V8<T> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)x[t * 8 + e];
  return r;
}

// Row of ND*32 columns from ND accumulators (lane (c, g): column c of the
// transposed product, rows crow(r, g)), times mul, rounded to T.
template <class T, int ND = 4>
__device__ __forceinline__ void store_row4x4(T* rowp, const f32x16* acc, float mul, int g) {
#pragma unroll
  for (int db = 0; db < ND; ++db)
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
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);
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
  int kb, bh;  // causal: lowest key blocks (most work) first
  xcd_block(nkb, CAUSAL, kb, bh);
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
  // K and V live in accumulator registers (see dkdv_pipe_d128).
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    asm("" : "+a"(kf[ks]));
    asm("" : "+a"(vf[ks]));
  }

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

// ------------------------------------------- dK / dV, software-pipelined
// The same work as dkdv_f16_d128 with 128-query tiles in the swizzled layout,
// rearranged so that the LDS reads of one 32-query block overlap the MFMAs of
// another:
//   * Q and dO tiles go from global memory straight into LDS through buffer
//     loads with an LDS destination.  Lane i of a wave writes its 16 bytes at
//     the wave's LDS address + 16*i, so the swizzle is applied to the global
//     chunk each lane fetches; rows at or past Sq fall outside the buffer's
//     byte range and read as zero.  No staging registers are needed.
//   * The row-wise Q and dO fragments of the next block (of the next tile,
//     after the last block) are read under the current block's dP and dV
//     products, a block's transposed fragments and row statistics under its
//     S product and the previous block's dK product, and the softmax-gradient
//     arithmetic is spread over all four products (the phases are listed
//     above the tile body below).
//   * One barrier per tile, inside its last block: after it the buffer just
//     read is refilled with the tile after next, and the next tile's first
//     fragments are read from the other buffer.
//   * Only the tiles that straddle the causal diagonal carry masks.  Keys past
//     Sk are not masked: their dK and dV columns depend on nothing else and
//     are never stored.
// Needs 32-bit byte offsets: (Sq + 3*128) * row stride * 2 bytes < 2^31 for
// Q and dO, and a row stride of at least 128 elements (checked on the host).
// WPE: waves per SIMD the registers must allow (1, or 2 at D = 64: two
// workgroups per CU; the operands then stay in architectural registers).
template <class T, bool CAUSAL, int D = 128, int WPE = 1>
__global__ __launch_bounds__(256, WPE) void dkdv_pipe(BwdArgs a) {
  constexpr int BM = 128, NW = 4, BN = 32 * NW, NQB = BM / 32, TR = BM * D, BUF = 2 * TR;
  constexpr int NK = D / 16, ND = D / 32;  // k-steps of S and dP; column blocks of dK and dV
  // Per scheduling group (one MFMA each): LDS reads of phase 1, VALU.
  constexpr int kDs1 = (4 * ND + 8) / NK, kVa = 32 / NK;
  __shared__ __attribute__((aligned(1024))) T smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float lsd[2][2][BM];  // [buffer][LSE*log2e, -delta][row]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nkb = (a.Sk + BN - 1) / BN;
  int kb, bh;
  xcd_block(nkb, CAUSAL, kb, bh);
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* dobase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  const rsrc_t rq = make_rsrc(qbase, (int)((int64_t)a.Sq * a.q.ss * (int64_t)sizeof(T)));
  const rsrc_t rd = make_rsrc(dobase, (int)((int64_t)a.Sq * a.dout.ss * (int64_t)sizeof(T)));
  const float* lse = a.lse + (int64_t)bh * a.Sq;
  const float* dl = a.delta + (int64_t)bh * a.Sq;
  const int k0 = kb * BN, kw = k0 + w * 32, kj = kw + c;

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dk[i] = zero16(); dv[i] = zero16(); }
  const float cs = a.scale_log2;

  const int qstart = CAUSAL ? (max(0, k0 - a.coff) / BM) * BM : 0;
  const int ntiles = a.Sq > qstart ? (a.Sq - qstart + BM - 1) / BM : 0;
  // Tile t is wholly visible when its first query sees the block's last key:
  // qstart + t*BM + coff >= k0 + BN - 1.  The tiles before that carry masks.
  const int hidden = k0 + BN - 1 - a.coff - qstart;
  const int nmask = CAUSAL ? min(ntiles, hidden > 0 ? (hidden + BM - 1) / BM : 0) : 0;

  // LSE and delta of row (tile start + thread % 128), loaded raw and converted
  // when stored (see dkdv_f16_d128).
  float lsr = 0.f, dlr = 0.f;
  bool lrow = false;
  const unsigned lds0 = lds_addr(smem);
  const int qsb = (int)(a.q.ss * (int64_t)sizeof(T)), dsb = (int)(a.dout.ss * (int64_t)sizeof(T));
  const int qlo = dma_lane_off<NW, D>(qsb), dlo = dma_lane_off<NW, D>(dsb);
  auto issue_tile = [&](int t, int buf) {
    const int q0 = qstart + t * BM;
    const unsigned base = lds0 + (unsigned)(buf * BUF * (int)sizeof(T));
    tile_dma<BM, NW, D>(rq, base, qlo, qsb, q0);
    tile_dma<BM, NW, D>(rd, base + (unsigned)(TR * (int)sizeof(T)), dlo, dsb, q0);
    const int i = q0 + ((int)threadIdx.x & (BM - 1));
    lrow = i < a.Sq;
    lsr = lse[min(i, a.Sq - 1)];
    dlr = dl[min(i, a.Sq - 1)];
  };
  auto store_rows = [&](int t) {
    if ((int)threadIdx.x < BM) {
      lsd[t & 1][0][threadIdx.x] = (!lrow || lsr == -INFINITY) ? INFINITY : lsr * kLog2e;
      lsd[t & 1][1][threadIdx.x] = lrow ? -dlr : 0.f;
    }
  };

  // Pipeline state carried from 32-query block j-1 into block j.
  V8<T> qf[NK];        // Q rows of block j (operand of S)
  V8<T> of[NK];        // dO rows of block j (operand of dP)
  V8<T> qtp[2][ND];    // transposed Q of block j-1 (operand of dK)
  f32x16 pc, dpc;      // P and dP - delta of block j-1
  V8<T> sf0;           // dS of block j-1, rows of k-step 0, rounded
  pc = zero16();
  dpc = zero16();
#pragma unroll
  for (int e = 0; e < 8; ++e) sf0[e] = (T)0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int db = 0; db < ND; ++db) qtp[tt][db] = sf0;
  // The first tile's buffer loads go out before the K and V row loads, so
  // that the prologue waits for one memory round trip, not two.  (Loads
  // issued after them complete after them, so the compiler's own waits for
  // the rows, which do not count these loads, are conservative.)
  if (ntiles > 0) issue_tile(0, 0);
  V8<T> kf[NK], vf[NK];
  {
    const int kc = min(kj, a.Sk - 1);
    const T* krow = (const T*)a.k.p + b * a.k.sb + h * a.k.sh + (int64_t)kc * a.k.ss;
    const T* vrow = (const T*)a.v.p + b * a.v.sb + h * a.v.sh + (int64_t)kc * a.v.ss;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      kf[ks] = *reinterpret_cast<const V8<T>*>(krow + ks * 16 + g * 8);
      vf[ks] = *reinterpret_cast<const V8<T>*>(vrow + ks * 16 + g * 8);
    }
    // K and V stay in accumulator registers for the whole kernel: MFMAs read
    // their A and B operands from either file, so these 64 (D = 128)
    // registers cost no copies, and the architectural file keeps room for the
    // S and dP products and the dK and dV sums (this file is built with the
    // VGPR accumulator form of the MFMAs, so S and dP reach the
    // softmax-gradient arithmetic without a v_accvgpr_read per element).
    if constexpr (WPE == 1) {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        asm("" : "+a"(kf[ks]));
        asm("" : "+a"(vf[ks]));
      }
    }
  }
  if (ntiles > 0) {
    store_rows(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): rows and this wave's buffer loads are in
    __syncthreads();
    if (ntiles > 1) issue_tile(1, 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qf[ks] = frag_r_swz<T, D>(smem, 0, ks * 2);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) of[ks] = frag_r_swz<T, D>(smem + TR, 0, ks * 2);
  }

  // Rows of k-step tt of an accumulator (crow order) out of four float4 runs.
  auto sel = [](const float4* v, int r) {
    return r % 4 == 0 ? v[r / 4].x : r % 4 == 1 ? v[r / 4].y : r % 4 == 2 ? v[r / 4].z : v[r / 4].w;
  };

  // Tile t: its data is in cur, the next tile's in nxt.  Block j runs four
  // phases, each one scheduling region whose NK MFMAs (eight at D = 128,
  // four at D = 64) are interleaved with
  // the LDS reads and the VALU work listed for it (a wave issues only a few
  // VALU instructions per MFMA without stalling the matrix pipe, so the
  // softmax-gradient arithmetic is spread evenly over all four):
  //   1: S(j) = Q K^T        | read dO^T(j), LSE(j), delta(j) | dS(j-1), second half
  //   2: dK += dS(j-1)^T Q   | read Q^T(j)                    | P(j), first half
  //   3: dP(j) = dO V^T      | read Q rows(j+1)               | P(j), second half
  //   4: dV += P(j)^T dO     | read dO rows(j+1)              | dS(j), first half
  // Phase 2 holds the block's last reads of cur; the tile's barrier sits
  // between phases 3 and 4 of its last block (so those reads have phase 3 to
  // land before the barrier waits for them), and phase 4 of that block reads
  // the next tile's first Q and dO rows from nxt.
  auto tile = [&](auto masked, int t, T* cur, T* nxt) {
    constexpr bool MASKED = decltype(masked)::value;
    const int q0 = qstart + t * BM;
    const T* Qc = cur;
    const T* Dc = Qc + TR;
    const T* Qn = nxt;
    const float* Ls = lsd[t & 1][0];
    const float* Dl = lsd[t & 1][1];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qs = q0 + qb * 32;
      V8<T> dt[2][ND], qt[2][ND], sf1, pf0, pf1;
      float4 l4[4];
      f32x16 s = zero16(), dp, p;  // dp starts from -delta: dP - delta comes out of the MFMAs
      // ---- 1
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < ND; ++db) dt[tt][db] = frag_t_swz<T, D>(Dc, qb * 32, tt, db * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l4[i] = *reinterpret_cast<const float4*>(Ls + qb * 32 + i * 8 + g * 4);
        const float4 d = *reinterpret_cast<const float4*>(Dl + qb * 32 + i * 8 + g * 4);
        dp[i * 4 + 0] = d.x; dp[i * 4 + 1] = d.y; dp[i * 4 + 2] = d.z; dp[i * 4 + 3] = d.w;
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) s = Mfma<T>::mma(qf[ks], kf[ks], s);
      {
        f32x16 x;
#pragma unroll
        for (int r = 8; r < 16; ++r) x[r] = pc[r] * dpc[r];
        sf1 = cvt8<T>(x, 1);
      }
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kDs1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- 2
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < ND; ++db) qt[tt][db] = frag_t_swz<T, D>(Qc, qb * 32, tt, db * 32);
#pragma unroll
      for (int db = 0; db < ND; ++db) dk[db] = Mfma<T>::mma(qtp[0][db], sf0, dk[db]);
#pragma unroll
      for (int db = 0; db < ND; ++db) dk[db] = Mfma<T>::mma(qtp[1][db], sf1, dk[db]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[r], cs, -sel(l4, r)));
        if (MASKED && kj > qs + a.coff + crow(r, g)) p[r] = 0.f;
      }
      pf0 = cvt8<T>(p, 0);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- 3
      const T* nq = qb + 1 < NQB ? Qc : Qn;
      const int nr = ((qb + 1) % NQB) * 32;
      if (qb + 1 < NQB) {
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) qf[ks] = frag_r_swz<T, D>(nq, nr, ks * 2);
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        if constexpr (WPE == 1) asm("" : "+a"(of[ks]));  // dO rows are read into accumulator registers
        dp = Mfma<T>::mma(of[ks], vf[ks], dp);
      }
#pragma unroll
      for (int r = 8; r < 16; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[r], cs, -sel(l4, r)));
        if (MASKED && kj > qs + a.coff + crow(r, g)) p[r] = 0.f;
      }
      pf1 = cvt8<T>(p, 1);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (qb == NQB - 1) {
        // Every wave is done reading this buffer (its last reads, in phase 2,
        // had phase 3 to land): refill it with the tile after next, and
        // publish the next tile's data and row statistics.
        store_rows(t + 1);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile's buffer loads are in LDS
        __syncthreads();
        if (t + 2 < ntiles) issue_tile(t + 2, t & 1);
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) qf[ks] = frag_r_swz<T, D>(nq, nr, ks * 2);
      }
      // ---- 4
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) of[ks] = frag_r_swz<T, D>(nq + TR, nr, ks * 2);
#pragma unroll
      for (int db = 0; db < ND; ++db) dv[db] = Mfma<T>::mma(dt[0][db], pf0, dv[db]);
#pragma unroll
      for (int db = 0; db < ND; ++db) dv[db] = Mfma<T>::mma(dt[1][db], pf1, dv[db]);
      {
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 8; ++r) x[r] = p[r] * dp[r];
        sf0 = cvt8<T>(x, 0);
      }
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      pc = p;
      dpc = dp;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < ND; ++db) qtp[tt][db] = qt[tt][db];
    }
  };
  int t = 0;
  for (; t < nmask; ++t) tile(BoolTag<true>{}, t, smem + (t & 1) * BUF, smem + ((t + 1) & 1) * BUF);
  for (; t < ntiles; ++t) tile(BoolTag<false>{}, t, smem + (t & 1) * BUF, smem + ((t + 1) & 1) * BUF);
  // Drain: the second half of the last block's dS, and its dK product.
  if (ntiles > 0) {
    f32x16 x;
#pragma unroll
    for (int r = 8; r < 16; ++r) x[r] = pc[r] * dpc[r];
    const V8<T> sf1 = cvt8<T>(x, 1);
#pragma unroll
    for (int db = 0; db < ND; ++db) dk[db] = Mfma<T>::mma(qtp[0][db], sf0, dk[db]);
#pragma unroll
    for (int db = 0; db < ND; ++db) dk[db] = Mfma<T>::mma(qtp[1][db], sf1, dk[db]);
  }

  if (kj < a.Sk) {
    T* dkrow = (T*)a.dk.p + b * a.dk.sb + h * a.dk.sh + (int64_t)kj * a.dk.ss;
    T* dvrow = (T*)a.dv.p + b * a.dv.sb + h * a.dv.sh + (int64_t)kj * a.dv.ss;
    store_row4x4<T, ND>(dkrow, dk, a.scale, g);
    store_row4x4<T, ND>(dvrow, dv, 1.f, g);
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

// ------------------------------------------------ dQ, buffer loads into LDS
// dq_f16_d128 with 64-key tiles in the swizzled layout and 8 waves, with the
// K and V tiles loaded straight into LDS by buffer loads (no staging
// registers; keys at or past Sk read as zero and are masked).  Each 32-key
// block runs its 24 MFMAs (S, dP, dQ) in a pinned order with every LDS
// fragment read four MFMAs ahead of its use; the registers that read-ahead
// needs come from subtracting delta after the dP product (one more VALU
// instruction per element) instead of holding it splatted as the dP start
// value, and from a compile-time buffer parity (immediate LDS offsets).
// Needs the 31-bit offsets the dK/dV kernel needs, for K and V.
// NW waves of 32 query rows: 8, or 4 so that two workgroups share a CU and
// one's prologue and epilogue overlap the other's tiles (either way two waves
// per SIMD).  Head dim D = 128 or 64 (at 64: 12 MFMAs a block, same order).
template <class T, bool CAUSAL, int NW = 8, int D = 128>
__global__ __launch_bounds__(NW * 64, 2) void dq_pipe(BwdArgs a) {
  constexpr int BM = 32 * NW, BN = 64, NT = NW * 64, NKB = BN / 32;
  constexpr int TR = BN * D, BUF = 2 * TR;  // K rows, V rows
  constexpr int NK = D / 16, ND = D / 32;   // k-steps of S and dP; column blocks of dQ
  __shared__ __attribute__((aligned(1024))) T smem[2 * BUF];
  (void)NT;

  // The wave index in a scalar register: the per-wave causal skips and mask
  // tests below are then uniform branches.
  const int lane = threadIdx.x & 63, g = lane >> 5, c = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  const rsrc_t rk = make_rsrc(kbase, (int)((int64_t)a.Sk * a.k.ss * (int64_t)sizeof(T)));
  const rsrc_t rv = make_rsrc(vbase, (int)((int64_t)a.Sk * a.v.ss * (int64_t)sizeof(T)));
  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;
  const bool valid = qi < a.Sq;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  const unsigned lds0 = lds_addr(smem);
  const int ksb = (int)(a.k.ss * (int64_t)sizeof(T)), vsb = (int)(a.v.ss * (int64_t)sizeof(T));
  const int klo = dma_lane_off<NW, D>(ksb), vlo = dma_lane_off<NW, D>(vsb);
  auto issue_tile = [&](int t) {
    const unsigned base = lds0 + (unsigned)((t & 1) * BUF * (int)sizeof(T));
    tile_dma<BN, NW, D>(rk, base, klo, ksb, t * BN);
    tile_dma<BN, NW, D>(rv, base + (unsigned)(TR * (int)sizeof(T)), vlo, vsb, t * BN);
  };
  // The first tile's buffer loads go out before the row loads, so that the
  // prologue waits for one memory round trip, not two.  (The row loads
  // issued after them complete after them, so the compiler's own waits for
  // the rows, which do not count these loads, are conservative.)
  if (ntiles > 0) issue_tile(0);

  V8<T> qf[NK], df[NK];
  const int qc = min(qi, a.Sq - 1);
  {
    const T* qrow = (const T*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qc * a.q.ss;
    const T* drow =
        (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh + (int64_t)qc * a.dout.ss;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      qf[ks] = *reinterpret_cast<const V8<T>*>(qrow + ks * 16 + g * 8);
      df[ks] = *reinterpret_cast<const V8<T>*>(drow + ks * 16 + g * 8);
    }
  }
  // Rows past the end, and rows with no visible key (LSE = -inf), get P = 0.
  const float lse_n = valid ? a.lse[(int64_t)bh * a.Sq + qi] : INFINITY;
  const float lse2 = lse_n == -INFINITY ? INFINITY : lse_n * kLog2e;
  float dlt;
  if (a.fuse_delta) {
    // delta = rowsum(dO o O) of this row ("Triton FlashAttention": the
    // backward's preprocess), formed here from the dO fragments this lane
    // holds and the matching half of the O row, the other half coming from
    // lane c + 32; written for the dK/dV kernel, which runs after this one.
    const T* orow = (const T*)a.o.p + b * a.o.sb + h * a.o.sh + (int64_t)qc * a.o.ss;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const V8<T> of = *reinterpret_cast<const V8<T>*>(orow + ks * 16 + g * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)df[ks][e], (float)of[e], acc);
    }
    dlt = acc + xor32(acc);
    if (valid && g == 0) a.delta[(int64_t)bh * a.Sq + qi] = dlt;
    if (!valid) dlt = 0.f;
  } else {
    dlt = valid ? a.delta[(int64_t)bh * a.Sq + qi] : 0.f;
  }
  f32x16 dq[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dq[i] = zero16();
  const float cs = a.scale_log2;

  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): rows and this wave's first-tile loads are in
  __syncthreads();

  // Tile t reads buffer t & 1, a compile-time constant below (the loop is
  // unrolled by two from an even t), so LDS fragment addresses are per-lane
  // bases plus immediate offsets.
  auto tile = [&](auto parity, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    const int k0 = t * BN;
    const T* Kr = smem + P * BUF;
    const T* Vr = Kr + TR;
    // The other buffer was last read in tile t-1, before the barrier below.
    if (t + 1 < ntiles) issue_tile(t + 1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int ks0 = k0 + kb * 32;
      if (CAUSAL && ks0 > qw + a.coff + 31) continue;
      // Products in a fixed order, each LDS fragment read issued four MFMAs
      // ahead of its use: the reads go in the order of their uses (K rows
      // for S, V rows for dP, then the two halves of transposed K for dQ),
      // read j issued with product j - 4; only VALU, SALU and global loads
      // may be scheduled across the pinned order.
      constexpr int kPin = 0x2 | 0x4 | 0x20, kAhead = 4, kReads = 2 * NK + 2 * ND;
      V8<T> kf[NK], vf[NK], kt[2][ND];
      auto fetch = [&](int j) __attribute__((always_inline)) {
        if (j < NK) kf[j] = frag_r_swz<T, D>(Kr, kb * 32, j * 2);
        else if (j < 2 * NK) vf[j - NK] = frag_r_swz<T, D>(Vr, kb * 32, (j - NK) * 2);
        else if (j < 2 * NK + ND) kt[0][j - 2 * NK] = frag_t_swz<T, D>(Kr, kb * 32, 0, (j - 2 * NK) * 32);
        else if (j < kReads) kt[1][j - 2 * NK - ND] = frag_t_swz<T, D>(Kr, kb * 32, 1, (j - 2 * NK - ND) * 32);
      };
#pragma unroll
      for (int j = 0; j < kAhead; ++j) fetch(j);
      __builtin_amdgcn_sched_barrier(kPin);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        fetch(ks + kAhead);
        s = Mfma<T>::mma(kf[ks], qf[ks], s);
        __builtin_amdgcn_sched_barrier(kPin);
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        fetch(NK + ks + kAhead);
        dp = Mfma<T>::mma(vf[ks], df[ks], dp);
        __builtin_amdgcn_sched_barrier(kPin);
      }
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
      const V8<T> sf0 = cvt8<T>(s, 0), sf1 = cvt8<T>(s, 1);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        fetch(2 * NK + db + kAhead);
        dq[db] = Mfma<T>::mma(kt[0][db], sf0, dq[db]);
        __builtin_amdgcn_sched_barrier(kPin);
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        fetch(2 * NK + ND + db + kAhead);
        dq[db] = Mfma<T>::mma(kt[1][db], sf1, dq[db]);
        __builtin_amdgcn_sched_barrier(kPin);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile's buffer loads are in LDS
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    tile(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) tile(std::integral_constant<int, 1>{}, t + 1);
  }

  if (valid) {
    T* row = (T*)a.dq.p + b * a.dq.sb + h * a.dq.sh + (int64_t)qi * a.dq.ss;
    store_row4x4<T, ND>(row, dq, a.scale, g);
  }
}

// Byte offsets of every K and V row the buffer-load dQ kernel may address
// (up to 3 tiles past Sk) fit in 31 bits, and rows do not overlap.
bool dq_pipe_fits(const BwdArgs& a, int esize, int D = kD) {
  const int64_t lim = (int64_t)1 << 31;
  return a.k.ss >= D && a.v.ss >= D && ((int64_t)a.Sk + 3 * 64) * a.k.ss * esize < lim &&
         ((int64_t)a.Sk + 3 * 64) * a.v.ss * esize < lim;
}

template <class T, bool CAUSAL, int NW = 8, int D = 128>
hipError_t launch_dq_pipe(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (((int64_t)a.Sq + 32 * NW - 1) / (32 * NW)) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dq_pipe<T, CAUSAL, NW, D>),
                         dim3((unsigned)grid), dim3(NW * 64), args, 0, s);
}

// Byte offsets of every Q and dO row the pipelined dK/dV kernel may address
// (up to 3 tiles past Sq) fit in 31 bits, and rows do not overlap.
bool dkdv_pipe_fits(const BwdArgs& a, int esize, int D = kD) {
  const int64_t lim = (int64_t)1 << 31;
  return a.q.ss >= D && a.dout.ss >= D && ((int64_t)a.Sq + 3 * 128) * a.q.ss * esize < lim &&
         ((int64_t)a.Sq + 3 * 128) * a.dout.ss * esize < lim;
}

template <class T, bool CAUSAL, int D = 128, int WPE = 1>
hipError_t launch_dkdv_pipe(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (((int64_t)a.Sk + 127) / 128) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dkdv_pipe<T, CAUSAL, D, WPE>),
                         dim3((unsigned)grid), dim3(256), args, 0, s);
}

}  // namespace

// dQ variants: 0 = (BN 64, 8 waves), 1 = (BN 64, 4 waves), 2 = (BN 32, 8 waves);
// 3, 4 = (BN 32, 64; 8 waves) with swizzled single-copy K and V; 5 = variant
// 4 with buffer loads into LDS and dP starting from -delta (variant 4 runs
// instead where its 31-bit offsets do not reach every row).  (With 128-key
// tiles the staging registers push the non-causal kernel into spills.)
// 6 = variant 5 with 4 waves, 128 query rows per workgroup and two workgroups
// per CU (variant 1 runs instead where the offsets do not reach).
// Head dim 64: dq_pipe with 8 (variant 0) or 4 (variant 1) waves; where its
// offsets do not reach, the caller runs a generic entry.
int dq_fast_variants(int D) { return D == 128 ? 7 : D == 64 ? 2 : 0; }
TileCfg dq_fast_cfg(int v, int D) {
  if (D == 64) {
    const int nw = v == 1 ? 4 : 8;
    return TileCfg{32 * nw, 64, nw, 2 * 2 * 64 * 64 * 2};
  }
  const int bn = v == 2 || v == 3 ? 32 : 64, nw = v == 1 || v == 6 ? 4 : 8;
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
    case 5:
      if (!dq_pipe_fits(a, (int)sizeof(T))) return launch_dq_variant<T>(a, 4, causal, s);
      return causal ? launch_dq_pipe<T, true>(a, s) : launch_dq_pipe<T, false>(a, s);
    case 6:
      if (!dq_pipe_fits(a, (int)sizeof(T))) return launch_dq_variant<T>(a, 1, causal, s);
      return causal ? launch_dq_pipe<T, true, 4>(a, s) : launch_dq_pipe<T, false, 4>(a, s);
  }
  return hipErrorInvalidValue;
}
template <class T>
hipError_t launch_dq_variant64(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dq_pipe<T, true, 8, 64>(a, s) : launch_dq_pipe<T, false, 8, 64>(a, s);
    case 1: return causal ? launch_dq_pipe<T, true, 4, 64>(a, s) : launch_dq_pipe<T, false, 4, 64>(a, s);
  }
  return hipErrorInvalidValue;
}
// dQ variants 5 and 6 (D = 128) and every D = 64 variant run dq_pipe where
// its 31-bit offsets reach every row: that kernel can form delta itself.
bool dq_fast_fuses_delta(const BwdArgs& a, int v, int dtype, int D) {
  const int es = dtype == 1 ? 4 : 2;
  if (D == 64) return dq_pipe_fits(a, es, 64);
  return (v == 5 || v == 6) && dq_pipe_fits(a, es);
}
bool dq_fast_runs(const BwdArgs& a, int dtype, int D) {
  (void)dtype;
  return D == 128 || dq_pipe_fits(a, 2, D);
}
hipError_t launch_dq_fast(const BwdArgs& a, int v, int dtype, int D, int causal, hipStream_t s) {
  if (D == 64) {
    if (dtype == 2) return launch_dq_variant64<bf16_t>(a, v, causal, s);
    return launch_dq_variant64<half_t>(a, v, causal, s);
  }
  if (dtype == 2) return launch_dq_variant<bf16_t>(a, v, causal, s);
  return launch_dq_variant<half_t>(a, v, causal, s);
}

// dK/dV variants: 0 = (BM 64, 4 waves), 1 = (BM 32, 4 waves), 2 = (BM 64,
// 4 waves, swizzled single-copy Q and dO), 3 = (BM 128, 4 waves, swizzled),
// 4 = variant 3 software-pipelined with buffer loads into LDS (variant 3 runs
// instead where its 31-bit offsets do not reach every row).  (With 8 waves, two per SIMD, the
// 32 keys' K, V, dK and dV no longer fit the 256 registers a wave then gets,
// and the compiler spills.)  5 = 128 keys over 8 waves, each 32-key slice
// split between a score wave (K, dV) and an accumulate wave (V, dK) that
// trade P through LDS, 64-query tiles in three buffers (fa_bwd_split.hip;
// variant 4 runs instead where its 31-bit offsets do not reach every row).
// Head dim 64: the software-pipelined kernel with one wave per SIMD (variant
// 0) or two (variant 1: two workgroups per CU, K, V and dO rows in
// architectural registers, 256 a wave); where its offsets do not reach, the
// caller runs a generic entry.
int dkdv_fast_variants(int D) { return D == 128 ? 6 : D == 64 ? 2 : 0; }
TileCfg dkdv_fast_cfg(int v, int D) {
  if (D == 64) return TileCfg{128, 128, 4, 2 * 2 * 128 * 64 * 2 + 2 * 2 * 128 * 4};
  if (v == 5) return TileCfg{64, 128, 8, dkdv_split_lds()};
  const int bm = v == 1 ? 32 : v >= 3 ? 128 : 64, nw = 4;
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
    case 4:
      if (!dkdv_pipe_fits(a, (int)sizeof(T))) return launch_dkdv_variant<T>(a, 3, causal, s);
      return causal ? launch_dkdv_pipe<T, true>(a, s) : launch_dkdv_pipe<T, false>(a, s);
    case 5:
      if (!dkdv_split_fits(a, (int)sizeof(T))) return launch_dkdv_variant<T>(a, 4, causal, s);
      return launch_dkdv_split(a, std::is_same<T, bf16_t>::value ? 2 : 0, causal, s);
  }
  return hipErrorInvalidValue;
}
template <class T>
hipError_t launch_dkdv_variant64(const BwdArgs& a, int v, int causal, hipStream_t s) {
  switch (v) {
    case 0: return causal ? launch_dkdv_pipe<T, true, 64>(a, s) : launch_dkdv_pipe<T, false, 64>(a, s);
    case 1: return causal ? launch_dkdv_pipe<T, true, 64, 2>(a, s) : launch_dkdv_pipe<T, false, 64, 2>(a, s);
  }
  return hipErrorInvalidValue;
}
bool dkdv_fast_runs(const BwdArgs& a, int dtype, int D) {
  (void)dtype;
  return D == 128 || dkdv_pipe_fits(a, 2, D);
}
hipError_t launch_dkdv_fast(const BwdArgs& a, int v, int dtype, int D, int causal, hipStream_t s) {
  if (D == 64) {
    if (dtype == 2) return launch_dkdv_variant64<bf16_t>(a, v, causal, s);
    return launch_dkdv_variant64<half_t>(a, v, causal, s);
  }
  if (dtype == 2) return launch_dkdv_variant<bf16_t>(a, v, causal, s);
  return launch_dkdv_variant<half_t>(a, v, causal, s);
}

}  // namespace fa
