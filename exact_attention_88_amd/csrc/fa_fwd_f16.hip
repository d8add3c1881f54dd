// Forward attention for 16-bit inputs (fp16, bf16) with head dim 128 (and,
// for the buffer-load kernel, 64) on gfx950: the tuned path.
//
// Same method as the generic forward kernel ("FlashAttention-2 from PyTorch to
// Triton": online softmax over streamed K/V tiles, one program per query tile;
// "Triton FlashAttention": exp2 on log2(e)-prescaled scores, causal block
// skipping, one LSE float per row), laid out for CDNA4:
//   * K and V tiles are double-buffered in LDS: the global loads of tile t+1
//     are issued into registers before tile t is computed and written to the
//     other buffer afterwards, so one barrier per tile suffices and HBM/L2
//     latency hides behind the MFMA work;
//   * each tile is read in one pattern only, so each gets the row padding
//     that makes that pattern bank-conflict free with plain base+offset
//     addressing: K rows (read row-wise, 16 rows x one 16-byte chunk per
//     ds_read_b128) are padded by 16 bytes, V rows (read transposed, 4 rows x
//     64 bytes per ds_read_b64_tr_b16 half-wave) by 64 bytes;
//   * the accumulator rescale is skipped when no row of the wave moved its
//     max, and in the pipelined kernel (the default) the max moves lazily and
//     K runs one tile ahead of V so that the scores of the next tile (MFMA)
//     overlap the softmax of the current one (VALU);
//   * workgroups are renumbered so that all query blocks of one (batch, head)
//     run on the same XCD (dispatch is round-robin over the 8 XCDs), letting
//     that XCD's L2 serve the shared K/V stream; causal blocks run longest
//     first.
#include <type_traits>

#include "fa_args.h"
#include "fa_common.h"
#include "fa_lds.h"

namespace fa {

namespace {

constexpr int kD = 128;

constexpr int kLSK = kD + 8;   // K tile row stride (halfs): 272 bytes
constexpr int kLSV = kD + 32;  // V tile row stride (halfs): 320 bytes

// Global -> register staging of a ROWS x 128 fp16 tile (16-byte chunks,
// PER per thread) and register -> padded LDS store.  Native vector types keep
// the staging in VGPRs.
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

// Row-wise operand fragment of the K tile: lane (c, g) gets row rbase + c,
// chunk kchunk + g.
template <class T>
__device__ __forceinline__ V8<T> frag_rows_k(const T* lds, int rbase, int kchunk) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const V8<T>*>(lds + (rbase + (lane & 31)) * kLSK +
                                      (kchunk + (lane >> 5)) * 8);
}

// Transposed operand fragment (see frag_tr in fa_common.h) of the V tile.
template <class T>
__device__ __forceinline__ V8<T> frag_tr_v(const T* lds, int rbase, int t, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 15;
  const int col = cbase + ((lane >> 4) & 1) * 16 + (j & 3) * 4;
  const int row = rbase + t * 16 + g * 4 + (j >> 2);
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const T* p0 = lds + row * kLSV + col;
  s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
  s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 8 * kLSV));
  V4<T> ah = __builtin_bit_cast(V4<T>, a), bh = __builtin_bit_cast(V4<T>, b);
  V8<T> r;
  r[0] = ah[0]; r[1] = ah[1]; r[2] = ah[2]; r[3] = ah[3];
  r[4] = bh[0]; r[5] = bh[1]; r[6] = bh[2]; r[7] = bh[3];
  return r;
}

template <class T, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_f16_d128(FwdArgs a) {
  constexpr int BM = 32 * NW, NT = NW * 64;
  constexpr int NKB = BN / 32;
  constexpr int TK = BN * kLSK, TV = BN * kLSV;
  __shared__ __attribute__((aligned(1024))) T smem[2 * TK + 2 * TV];  // K0 K1 V0 V1

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;

  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;

  V8<T> qf[8];
  {
    const T* qrow = qbase + (int64_t)min(qi, a.Sq - 1) * a.q.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const V8<T>*>(qrow + ks * 16 + g * 8);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): Q is resident before the tile loop

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;

  constexpr int PER = BN * 16 / NT;
  u32x4 kr[PER], vr[PER];
  tile_load<BN, NT>(kr, kbase, a.k.ss, 0, a.Sk);
  tile_load<BN, NT>(vr, vbase, a.v.ss, 0, a.Sk);
  tile_store<BN, NT, kLSK>(kr, smem);
  tile_store<BN, NT, kLSV>(vr, smem + 2 * TK);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const int buf = t & 1;
    const T* Ks = smem + buf * TK;
    const T* Vs = smem + 2 * TK + buf * TV;
    __syncthreads();
    const bool more = t + 1 < ntiles;
    if (more) {
      tile_load<BN, NT>(kr, kbase, a.k.ss, k0 + BN, a.Sk);
      tile_load<BN, NT>(vr, vbase, a.v.ss, k0 + BN, a.Sk);
    }
    if (!(CAUSAL && k0 > qw + a.coff + 31)) {
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        V8<T> kf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kf[ks] = frag_rows_k(Ks, kb * 32, ks * 2);
        s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          s[kb] = Mfma<T>::mma(kf[ks], qf[ks], s[kb]);
      }
      if ((k0 + BN > a.Sk) || (CAUSAL && k0 + BN - 1 > qw + a.coff)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + crow(r, g);
            if (key >= a.Sk || (CAUSAL && key > qi + a.coff)) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, xor32(mx));
      const float mnew = fmaxf(m, mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float mc = muse * cs;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], cs, -mc));
          s[kb][r] = p;
          rs += p;
        }
      if (__any(mnew != m)) {
        const float alpha = fast_exp2((m - muse) * cs);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      lsum += rs;
      m = mnew;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          V8<T> vf[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) vf[db] = frag_tr_v(Vs, kb * 32, tt, db * 32);
          V8<T> pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (T)s[kb][tt * 8 + e];
#pragma unroll
          for (int db = 0; db < 4; ++db)
            oacc[db] = Mfma<T>::mma(vf[db], pf, oacc[db]);
        }
    }
    if (more) {
      tile_store<BN, NT, kLSK>(kr, smem + (buf ^ 1) * TK);
      tile_store<BN, NT, kLSV>(vr, smem + 2 * TK + (buf ^ 1) * TV);
    }
  }

  const float ltot = lsum + xor32(lsum);
  if (qi < a.Sq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // no visible key: O = 0, LSE = -inf
    T* orow = (T*)a.o.p + b * a.o.sb + h * a.o.sh + (int64_t)qi * a.o.ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        V4<T> o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[db][r4 * 4 + e] * inv);
        *reinterpret_cast<V4<T>*>(orow + db * 32 + r4 * 8 + g * 4) = o4;
      }
    if (g == 0)
      a.lse[(int64_t)bh * a.Sq + qi] =
          ltot > 0.f ? __builtin_fmaf(a.scale, m, fast_log2(ltot) * kLn2) : -INFINITY;
  }
}

// Pair-wise combine across the two half-waves (lanes l and l ^ 32) with
// gfx950's v_permlane32_swap: a VALU exchange instead of an LDS permute.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scores of one tile for one wave without scheduling constraints.
template <int NKB, class T>
__device__ __forceinline__ void scores_free(f32x16* s, const T* Ks, const V8<T>* qf) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    V8<T> kf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = frag_rows_k(Ks, kb * 32, ks * 2);
    s[kb] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      s[kb] = Mfma<T>::mma(kf[ks], qf[ks], s[kb]);
  }
}

// Scores with a fixed order of LDS reads and MFMAs: the first 32-key block's
// eight K fragments are read up front, and each score MFMA is followed by one
// fragment read of the next block, so every read has several MFMAs' time to
// land.  The sched_barrier fences pin that order and let only VALU, SALU and
// global loads (the softmax of the previous tile, address arithmetic) move
// across, into the gaps.
template <int NKB, class T>
__device__ __forceinline__ void scores_ordered(f32x16* s, const T* Ks, const V8<T>* qf) {
  constexpr int kFloat = 0x2 | 0x4 | 0x20;  // VALU, SALU, VMEM read
  V8<T> kf[2][8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kf[0][ks] = frag_rows_k(Ks, 0, ks * 2);
  __builtin_amdgcn_sched_barrier(kFloat);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s[kb] = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s[kb] = Mfma<T>::mma(kf[kb & 1][ks], qf[ks], s[kb]);
      if (kb + 1 < NKB) kf[(kb + 1) & 1][ks] = frag_rows_k(Ks, (kb + 1) * 32, ks * 2);
      __builtin_amdgcn_sched_barrier(kFloat);
    }
  }
}

// O^T += V^T P^T for one tile with the same pinned order: the transposed V
// fragments of the first 16-key step are read up front, and each MFMA is
// followed by the reads of one fragment of the next step.
template <int NKB, class T>
__device__ __forceinline__ void pv_ordered(f32x16* oacc, const T* Vs, const f32x16* p,
                                           const V8<T>* vf0) {
  constexpr int kFloat = 0x2 | 0x4 | 0x20 | 0x200;  // VALU, SALU, VMEM read, DS write
  constexpr int NS = NKB * 2;                       // 16-key steps per tile
  V8<T> vf[2][4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vf[0][db] = vf0[db];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int kb = st >> 1, tt = st & 1;
    V8<T> pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (T)p[kb][tt * 8 + e];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      oacc[db] = Mfma<T>::mma(vf[st & 1][db], pf, oacc[db]);
      if (st + 1 < NS)
        vf[(st + 1) & 1][db] = frag_tr_v(Vs, ((st + 1) >> 1) * 32, (st + 1) & 1, db * 32);
      __builtin_amdgcn_sched_barrier(kFloat);
    }
  }
}

// A row's running max is raised only when a tile's scores exceed it by more
// than this many powers of two; until then probabilities are taken against
// the stale max and stay below 2^kLazy (exact: the output's numerator and
// denominator share that max, and 2^8 is far inside fp16 and fp32 range).
constexpr float kLazy = 8.f;

// Pipelined kernel.  K runs one tile ahead of V through LDS, so iteration t
// holds the scores S(t+1) (MFMA) and the softmax of tile t (VALU), which do
// not depend on each other: iteration t loads K(t+2) and V(t+1) from HBM,
// computes S(t+1) from K(t+1), softmax(t), then O += P(t) V(t), and stores
// the staged tiles into the buffers that held K(t) and V(t-1).  One barrier
// per tile.  The steady-state iteration is one basic block apart from the
// rare rescale: the global loads and LDS stores are unconditional (rows are
// clamped in bounds; what the last iterations stage is never read), masks live
// in a second copy of the loop that runs only the diagonal and ragged-tail
// tiles, the running max moves lazily (kLazy) so the rescale branch is rarely
// taken, and the half-wave max and sum use a VALU lane swap.
// ORDERED pins the read/MFMA order (scores_ordered, pv_ordered) and reads the
// first V fragments before the scores.
template <class T, int BN, int NW, bool CAUSAL, bool ORDERED>
__global__ __launch_bounds__(NW * 64, 2) void fwd_f16_d128_pipe(FwdArgs a) {
  constexpr int BM = 32 * NW, NT = NW * 64;
  constexpr int NKB = BN / 32;
  constexpr int TK = BN * kLSK, TV = BN * kLSV;
  __shared__ __attribute__((aligned(1024))) T smem[2 * TK + 2 * TV];  // K0 K1 V0 V1

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;

  const int q0 = qb * BM, qi = q0 + w * 32 + c;

  V8<T> qf[8];
  {
    const T* qrow = qbase + (int64_t)min(qi, a.Sq - 1) * a.q.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const V8<T>*>(qrow + ks * 16 + g * 8);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): Q is resident before the tile loop

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  // Tiles [0, nfull) hold no key past the end and, causally, no key after the
  // block's first query: no wave of the block masks them.  Every wave runs
  // every tile of its block: a tile entirely after a wave's rows is fully
  // masked (P = 0) and changes nothing.
  const int nfull = min(ntiles, (CAUSAL ? max(0, min(a.Sk, q0 + a.coff + 1)) : a.Sk) / BN);

  constexpr int PER = BN * 16 / NT;
  u32x4 kr[PER], vr[PER];
  tile_load<BN, NT>(kr, kbase, a.k.ss, 0, a.Sk);
  tile_load<BN, NT>(vr, vbase, a.v.ss, 0, a.Sk);
  tile_store<BN, NT, kLSK>(kr, smem);
  tile_store<BN, NT, kLSV>(vr, smem + 2 * TK);
  tile_load<BN, NT>(kr, kbase, a.k.ss, BN, a.Sk);
  tile_store<BN, NT, kLSK>(kr, smem + TK);
  __syncthreads();
  f32x16 scur[NKB];
  scores_free<NKB>(scur, smem, qf);
  // Iteration 0 overwrites K buffer 0: every wave must have read it first.
  __syncthreads();

  // Iteration t: stage K(t+2) and V(t+1), S(t+1) from K buffer (t+1)&1,
  // softmax(t), O += P(t) V(t) from V buffer t&1, then store K(t+2) into K
  // buffer t&1 (last read by S(t), one barrier ago) and V(t+1) into V buffer
  // (t+1)&1 (last read by PV(t-1), one barrier ago).
  auto step = [&](int t, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int k0 = t * BN;
    tile_load<BN, NT>(kr, kbase, a.k.ss, k0 + 2 * BN, a.Sk);
    tile_load<BN, NT>(vr, vbase, a.v.ss, k0 + BN, a.Sk);
    f32x16 snxt[NKB];
    const T* Vs = smem + 2 * TK + (t & 1) * TV;
    const T* Kn = smem + ((t + 1) & 1) * TK;
    V8<T> vf0[4];
    if constexpr (ORDERED) {
#pragma unroll
      for (int db = 0; db < 4; ++db) vf0[db] = frag_tr_v(Vs, 0, 0, db * 32);
      scores_ordered<NKB>(snxt, Kn, qf);
    } else {
      scores_free<NKB>(snxt, Kn, qf);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + crow(r, g);
          if (key >= a.Sk || (CAUSAL && key > qi + a.coff)) scur[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb][r]);
    mx = max_xor32(mx);
    // m = -inf and a finite mx give +inf > kLazy: the first scores always
    // raise the max.  Both -inf (a row with no key yet) give NaN: no raise.
    const bool raise = (mx - m) * cs > kLazy;
    const float mnew = raise ? mx : m;
    const float mc = (mnew == -INFINITY ? 0.f : mnew) * cs;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(scur[kb][r], cs, -mc));
        scur[kb][r] = p;
        rs += p;
      }
    if (__any(raise)) {
      const float alpha = raise ? fast_exp2((m - mnew) * cs) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    lsum += rs;
    m = mnew;
    if constexpr (ORDERED) {
      pv_ordered<NKB>(oacc, Vs, scur, vf0);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          V8<T> vf[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) vf[db] = frag_tr_v(Vs, kb * 32, tt, db * 32);
          V8<T> pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (T)scur[kb][tt * 8 + e];
#pragma unroll
          for (int db = 0; db < 4; ++db)
            oacc[db] = Mfma<T>::mma(vf[db], pf, oacc[db]);
        }
    }
    tile_store<BN, NT, kLSK>(kr, smem + (t & 1) * TK);
    tile_store<BN, NT, kLSV>(vr, smem + 2 * TK + ((t + 1) & 1) * TV);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) scur[kb] = snxt[kb];
  };
  int t = 0;
  for (; t < nfull; ++t) step(t, std::false_type{});
  for (; t < ntiles; ++t) step(t, std::true_type{});

  const float ltot = add_xor32(lsum);
  if (qi < a.Sq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // no visible key: O = 0, LSE = -inf
    T* orow = (T*)a.o.p + b * a.o.sb + h * a.o.sh + (int64_t)qi * a.o.ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        V4<T> o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[db][r4 * 4 + e] * inv);
        *reinterpret_cast<V4<T>*>(orow + db * 32 + r4 * 8 + g * 4) = o4;
      }
    if (g == 0)
      a.lse[(int64_t)bh * a.Sq + qi] =
          ltot > 0.f ? __builtin_fmaf(a.scale, m, fast_log2(ltot) * kLn2) : -INFINITY;
  }
}


// Pipelined kernel with buffer loads into LDS.  The method and the K-ahead
// pipeline are those of fwd_f16_d128_pipe; what changes is how the work is
// laid out over the instruction stream, since a wave issues only a few VALU
// instructions per MFMA without stalling the matrix pipe and the softmax is
// VALU-heavy:
//   * K and V tiles are loaded straight from global memory into one swizzled
//     copy each (no staging registers, no per-tile address arithmetic beyond a
//     32-bit offset; keys at or past Sk read as zero and are masked);
//   * the loop is unrolled by two, so the scores of the current and the next
//     tile swap roles without register copies;
//   * tile t runs as four scheduling regions, each with eight MFMAs
//     interleaved with the LDS reads and VALU work listed for it:
//       1: S(t+1), first 32 keys    | read V^T(t), first 32 keys  | P(t), first 32 keys
//       2: O += P V(t), first half  | read K(t+1), second 32 keys | P(t), next 16 keys; row sum
//       3: S(t+1), second 32 keys   | read V^T(t), second 32 keys | P(t), last 16 keys; row sum
//       4: O += P V(t), second half | read K(t+2), first 32 keys  | mask and row max of S(t+1)
//     with the tile's barrier between regions 3 and 4: it publishes K(t+2)
//     and V(t+1) and frees the buffers of K(t+1) and V(t), which are refilled
//     with K(t+3) and V(t+2) right after it.
// Needs 31-bit byte offsets for every K and V row below Sk + 4*64 and a row
// stride of at least D elements (checked on the host).
// NW waves of 32 query rows (8, or 4 so that two workgroups share a CU and
// one's prologue and epilogue overlap the other's tiles; either way two
// waves per SIMD).
// Head dim D = 128 or 64.  At D = 64 a tile holds half the MFMAs (QK^T takes
// four k-steps, O two column blocks) for the same softmax work, so each of
// the four regions interleaves four MFMAs with twice the VALU per MFMA.
template <class T, bool CAUSAL, int NW = 8, int D = 128>
__global__ __launch_bounds__(NW * 64, 2) void fwd_dma(FwdArgs a) {
  static_assert(NW == 4 || NW == 8, "buffer loads move whole multiples of 16 rows");
  static_assert(D == 128 || D == 64, "tuned head dims");
  constexpr int BM = 32 * NW, BN = 64, TR = BN * D;
  constexpr int NK = D / 16;  // k-steps of QK^T (and K fragments per 32 keys)
  constexpr int ND = D / 32;  // 32-column blocks of O
  // Per scheduling group (one MFMA each): exponentials of regions 1 and 2/3,
  // other VALU.
  constexpr int kTr1 = 16 / NK, kTr2 = 8 / NK, kVa = 24 / NK;
  __shared__ __attribute__((aligned(1024))) T smem[4 * TR];  // K0 K1 V0 V1

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);
  if (CAUSAL) qb = nqb - 1 - qb;
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  const swzl::rsrc_t rk = swzl::make_rsrc(kbase, (int)((int64_t)a.Sk * a.k.ss * (int64_t)sizeof(T)));
  const swzl::rsrc_t rv = swzl::make_rsrc(vbase, (int)((int64_t)a.Sk * a.v.ss * (int64_t)sizeof(T)));

  const int q0 = qb * BM, qi = q0 + w * 32 + c;

  V8<T> qf[NK];
  {
    const T* qrow = qbase + (int64_t)min(qi, a.Sq - 1) * a.q.ss;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qf[ks] = *reinterpret_cast<const V8<T>*>(qrow + ks * 16 + g * 8);
  }
  // Q resident before any buffer load into LDS is issued (the compiler does
  // not count those).
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) oacc[i] = zero16();
  float m = -INFINITY, lsum = 0.f, mc = 0.f;
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  // Tiles [0, nfull) hold no key past the end and, causally, no key after the
  // block's first query: their scores need no mask.
  const int nfull = min(ntiles, (CAUSAL ? max(0, min(a.Sk, q0 + a.coff + 1)) : a.Sk) / BN);

  // Buffer of tile t's K or V: chosen by t's parity, which is a compile-time
  // constant in the loop below (unrolled by two from an even t), so that LDS
  // addresses are a per-lane base plus constant offsets.
  auto kbuf = [&](int par) { return smem + (par & 1) * TR; };
  auto vbuf = [&](int par) { return smem + 2 * TR + (par & 1) * TR; };
  const unsigned lds0 = swzl::lds_addr(smem);
  const int ksb = (int)(a.k.ss * (int64_t)sizeof(T)), vsb = (int)(a.v.ss * (int64_t)sizeof(T));
  const int klo = swzl::dma_lane_off<NW, D>(ksb), vlo = swzl::dma_lane_off<NW, D>(vsb);
  auto dma_k = [&](int t, int par) {
    swzl::tile_dma<BN, NW, D>(rk, lds0 + (unsigned)((par & 1) * TR * (int)sizeof(T)), klo, ksb, t * BN);
  };
  auto dma_v = [&](int t, int par) {
    swzl::tile_dma<BN, NW, D>(rv, lds0 + (unsigned)((2 + (par & 1)) * TR * (int)sizeof(T)), vlo, vsb, t * BN);
  };
  auto kfrag = [](const T* buf, int rbase, int kchunk) { return swzl::frag_r_swz<T, D>(buf, rbase, kchunk); };
  auto vfrag = [](const T* buf, int rbase, int tt, int cbase) {
    return swzl::frag_t_swz<T, D>(buf, rbase, tt, cbase);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's buffer loads are in LDS
    __syncthreads();
  };
  // Mask tile u's scores (keys past Sk or, causally, after the row), take the
  // row max and move the running max if it grew by more than 2^kLazy,
  // rescaling O and the row sum.
  // Max of one accumulator's 16 values as a balanced tree of v_max3 (a short
  // dependency chain instead of 16 in a row).
  auto max16 = [](const f32x16& x) {
    const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
    const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
    const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
    return fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15]));
  };
  auto mask = [&](f32x16* sc, int u) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = u * BN + kb * 32 + crow(r, g);
        if (key >= a.Sk || (CAUSAL && key > qi + a.coff)) sc[kb][r] = -INFINITY;
      }
  };
  // Move the running max to mx (this half-wave's max of the tile) if it grew
  // by more than 2^kLazy, rescaling O and the row sum.
  auto update = [&](float mx) {
    mx = max_xor32(mx);
    // m = -inf and a finite mx give +inf > kLazy: the first scores always
    // raise the max.  Both -inf (a row with no key yet) give NaN: no raise.
    const bool raise = (mx - m) * cs > kLazy;
    const float mnew = raise ? mx : m;
    if (__any(raise)) {
      const float alpha = raise ? fast_exp2((m - mnew) * cs) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    m = mnew;
    mc = (mnew == -INFINITY ? 0.f : mnew) * cs;
  };
  auto rowmax = [&](f32x16* sc, int u) {
    if (u >= nfull) mask(sc, u);
    update(fmaxf(max16(sc[0]), max16(sc[1])));
  };

  f32x16 sa[2], sb[2];
  V8<T> kf[NK];
  if (ntiles > 0) {
    dma_k(0, 0);
    dma_k(1, 1);
    dma_v(0, 0);
    barrier();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) kf[ks] = kfrag(kbuf(0), kb * 32, ks * 2);
      sa[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) sa[kb] = Mfma<T>::mma(kf[ks], qf[ks], sa[kb]);
    }
    __syncthreads();  // every wave has read K(0)'s buffer
    dma_k(2, 0);
    dma_v(1, 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) kf[ks] = kfrag(kbuf(1), 0, ks * 2);
    rowmax(sa, 0);
  }

  // Causal: the last key tile any row of this wave sees.  Past it the wave
  // has nothing to compute (its probabilities of later tiles are all zero),
  // so for those tiles it only joins the barrier and issues its share of the
  // loads (the second loop below).
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int ulast = CAUSAL ? (q0 + wv * 32 + 31 + a.coff) / BN : 0x7fffffff;

  // Tile t: scores S(t) in sc (row max taken), kf holds K(t+1)'s first 32
  // keys; K(t+1) and V(t) are in LDS, K(t+2) and V(t+1) are being loaded.
  auto step = [&](auto parity, int t, f32x16* sc, f32x16* sn) {
    constexpr int P = decltype(parity)::value;  // t & 1
    const T* Kn = kbuf(P + 1);
    const T* Vc = vbuf(P);
    V8<T> vt[2][ND], pf[2][2];
    float rs = 0.f;
    // ---- 1
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < ND; ++db) vt[tt][db] = vfrag(Vc, 0, tt, db * 32);
    sn[0] = zero16();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) sn[0] = Mfma<T>::mma(kf[ks], qf[ks], sn[0]);
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[0][r] = fast_exp2(__builtin_fmaf(sc[0][r], cs, -mc));
    pf[0][0] = frag_from_acc<T>(sc[0], 0);
    pf[0][1] = frag_from_acc<T>(sc[0], 1);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, kTr1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- 2
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) kf[ks] = kfrag(Kn, 32, ks * 2);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] = Mfma<T>::mma(vt[tt][db], pf[0][tt], oacc[db]);
#pragma unroll
    for (int r = 0; r < 8; ++r) sc[1][r] = fast_exp2(__builtin_fmaf(sc[1][r], cs, -mc));
    pf[1][0] = frag_from_acc<T>(sc[1], 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) rs += sc[0][r];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, kTr2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- 3
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < ND; ++db) vt[tt][db] = vfrag(Vc, 32, tt, db * 32);
    sn[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) sn[1] = Mfma<T>::mma(kf[ks], qf[ks], sn[1]);
#pragma unroll
    for (int r = 8; r < 16; ++r) sc[1][r] = fast_exp2(__builtin_fmaf(sc[1][r], cs, -mc));
    pf[1][1] = frag_from_acc<T>(sc[1], 1);
#pragma unroll
    for (int r = 0; r < 16; ++r) rs += sc[1][r];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, kTr2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Publish K(t+2) and V(t+1); the buffers of K(t+1) and V(t) are free.
    barrier();
    dma_k(t + 3, P + 1);
    dma_v(t + 2, P);
    // ---- 4
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) kf[ks] = kfrag(kbuf(P), 0, ks * 2);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] = Mfma<T>::mma(vt[tt][db], pf[1][tt], oacc[db]);
    lsum += rs;
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < ntiles) rowmax(sn, t + 1);
  };
  const int tc = CAUSAL ? min(ntiles, max(0, ulast + 1)) : ntiles;
  for (int t = 0; t < tc; t += 2) {
    step(std::integral_constant<int, 0>{}, t, sa, sb);
    if (t + 1 < tc) step(std::integral_constant<int, 1>{}, t + 1, sb, sa);
  }
  for (int t = tc; t < ntiles; ++t) {  // causal: past this wave's last visible key
    barrier();
    dma_k(t + 3, t + 1);
    dma_v(t + 2, t);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no buffer load outlives the workgroup

  const float ltot = add_xor32(lsum);
  if (qi < a.Sq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // no visible key: O = 0, LSE = -inf
    T* orow = (T*)a.o.p + b * a.o.sb + h * a.o.sh + (int64_t)qi * a.o.ss;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        V4<T> o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[db][r4 * 4 + e] * inv);
        *reinterpret_cast<V4<T>*>(orow + db * 32 + r4 * 8 + g * 4) = o4;
      }
    if (g == 0)
      a.lse[(int64_t)bh * a.Sq + qi] =
          ltot > 0.f ? __builtin_fmaf(a.scale, m, fast_log2(ltot) * kLn2) : -INFINITY;
  }
}

template <class Kernel>
hipError_t launch_k(Kernel* k, int BM, int threads, const FwdArgs& a, hipStream_t s) {
  const int64_t grid = (((int64_t)a.Sq + BM - 1) / BM) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid), dim3(threads),
                         args, 0, s);
}

template <class T, int BN, int NW, bool ORDERED>
hipError_t launch_pipe(const FwdArgs& a, int causal, hipStream_t s) {
  return causal ? launch_k(&fwd_f16_d128_pipe<T, BN, NW, true, ORDERED>, 32 * NW, NW * 64, a, s)
                : launch_k(&fwd_f16_d128_pipe<T, BN, NW, false, ORDERED>, 32 * NW, NW * 64, a, s);
}

template <class T, int BN, int NW>
hipError_t launch_plain(const FwdArgs& a, int causal, hipStream_t s) {
  return causal ? launch_k(&fwd_f16_d128<T, BN, NW, true>, 32 * NW, NW * 64, a, s)
                : launch_k(&fwd_f16_d128<T, BN, NW, false>, 32 * NW, NW * 64, a, s);
}

// Byte offsets of every K and V row the buffer-load kernel may address fit in
// 31 bits, and rows do not overlap.  The last loads reach K tile ntiles + 2,
// whose rows end below Sk + 4*64.
bool fwd_dma_fits(const FwdArgs& a, int esize, int D) {
  const int64_t lim = (int64_t)1 << 31;
  return a.k.ss >= D && a.v.ss >= D && ((int64_t)a.Sk + 4 * 64) * a.k.ss * esize < lim &&
         ((int64_t)a.Sk + 4 * 64) * a.v.ss * esize < lim;
}

template <class T>
hipError_t launch_variant(const FwdArgs& a, int variant, int causal, hipStream_t s) {
  const bool fits = fwd_dma_fits(a, (int)sizeof(T), kD);
  switch (variant) {
    case 0: return launch_pipe<T, 64, 8, true>(a, causal, s);
    case 1: return launch_pipe<T, 64, 8, false>(a, causal, s);
    case 2: return launch_plain<T, 64, 8>(a, causal, s);
    case 3: return launch_plain<T, 64, 4>(a, causal, s);
    case 4:
      if (!fits) return launch_pipe<T, 64, 8, true>(a, causal, s);
      return causal ? launch_k(&fwd_dma<T, true>, 256, 512, a, s)
                    : launch_k(&fwd_dma<T, false>, 256, 512, a, s);
    case 5:
      if (!fits) return launch_plain<T, 64, 4>(a, causal, s);
      return causal ? launch_k(&fwd_dma<T, true, 4>, 128, 256, a, s)
                    : launch_k(&fwd_dma<T, false, 4>, 128, 256, a, s);
  }
  return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_variant64(const FwdArgs& a, int variant, int causal, hipStream_t s) {
  switch (variant) {
    case 0:
      return causal ? launch_k(&fwd_dma<T, true, 8, 64>, 256, 512, a, s)
                    : launch_k(&fwd_dma<T, false, 8, 64>, 256, 512, a, s);
    case 1:
      return causal ? launch_k(&fwd_dma<T, true, 4, 64>, 128, 256, a, s)
                    : launch_k(&fwd_dma<T, false, 4, 64>, 128, 256, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Head dim 128 variants (BN keys per tile, waves): pipelined 0 = (64, 8,
// ordered), 1 = (64, 8); plain 2 = (64, 8), 3 = (64, 4); 4 = pipelined
// (64, 8) with buffer loads into LDS (variant 0 runs instead where its 31-bit
// offsets do not reach every row); 5 = variant 4 with 4 waves, 128 query rows
// per workgroup and two workgroups per CU (variant 3 runs instead where the
// offsets do not reach).
// Head dim 64: the buffer-load kernel with 8 (variant 0) or 4 (variant 1)
// waves; where its offsets do not reach, the caller runs a generic entry.
int fwd_fast_variants(int D) { return D == 128 ? 6 : D == 64 ? 2 : 0; }

TileCfg fwd_fast_cfg(int v, int D) {
  if (D == 64) {
    const int nw = v == 1 ? 4 : 8;
    return TileCfg{32 * nw, 64, nw, 4 * 64 * 64 * 2};
  }
  const int nw = v == 3 || v == 5 ? 4 : 8;
  if (v >= 4) return TileCfg{32 * nw, 64, nw, 4 * 64 * kD * 2};
  return TileCfg{32 * nw, 64, nw, 2 * 64 * (kLSK + kLSV) * 2};
}

bool fwd_fast_runs(const FwdArgs& a, int dtype, int D) {
  (void)dtype;
  return D == 128 || fwd_dma_fits(a, 2, D);
}

hipError_t launch_fwd_fast(const FwdArgs& a, int variant, int dtype, int D, int causal, hipStream_t s) {
  if (D == 64) {
    if (dtype == 2) return launch_variant64<bf16_t>(a, variant, causal, s);
    return launch_variant64<half_t>(a, variant, causal, s);
  }
  if (dtype == 2) return launch_variant<bf16_t>(a, variant, causal, s);
  return launch_variant<half_t>(a, variant, causal, s);
}

}  // namespace fa
