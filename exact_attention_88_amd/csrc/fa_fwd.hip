// Forward attention kernel for gfx950.
//
// Method ("FlashAttention-2 from PyTorch to Triton", the forward pass and its
// Triton kernel; "Triton FlashAttention", the forward kernel description):
// one workgroup per (query block, batch*head); each wave owns 32 query rows
// whose Q fragments stay in registers; K and V tiles of BN keys stream
// through LDS; scores are computed transposed, S^T = K Q^T, so that each lane
// owns one query row (row statistics need one cross-half exchange) and the
// probability tile can be fed straight back as the B operand of
// O^T += V^T P^T.  The online softmax keeps fp32 running max m and sum l in
// log2 units (scores prescaled by scale*log2(e) with one FMA, exp2), rescales
// the accumulator when the max moves, divides by l once at the end and writes
// LSE = ln2 * (m + log2 l).  Causal key blocks above a wave's diagonal are
// skipped; masks are evaluated only on diagonal and ragged tiles.
#include "fa_args.h"
#include "fa_common.h"

namespace fa {

namespace {

constexpr int kLdsMax = 65536;

// Keys per tile, waves, and K/V buffers in LDS (1: load then compute, two
// barriers per tile; 2: the next tile's global reads are issued into
// registers before the current tile is computed and stored to the other
// buffer after it, one barrier per tile).  New configurations go at the end
// so that the ids of the existing ones do not move.
struct FwdTile { int bn, nw, nb; };
constexpr FwdTile kTilesH[] = {{64, 4, 1}, {32, 4, 1}, {64, 2, 1}, {64, 8, 1}, {128, 4, 1},
                               {64, 4, 2}, {32, 4, 2}, {64, 8, 2}};
constexpr FwdTile kTilesF[] = {{32, 4, 1}, {32, 2, 1}, {64, 4, 1}, {32, 8, 1}, {32, 4, 2}, {32, 2, 2}};
constexpr int kNumH = sizeof(kTilesH) / sizeof(kTilesH[0]);
constexpr int kNumF = sizeof(kTilesF) / sizeof(kTilesF[0]);

constexpr int lds_bytes(int esize, int D, int bn, int nb) {
  return nb * 2 * bn * ((D < 32 ? 32 : D) + 16 / esize) * esize;
}
constexpr FwdTile tile_at(int dt, int i) { return dt == 0 ? kTilesH[i] : kTilesF[i]; }
constexpr int num_tiles_raw(int dt) { return dt == 0 ? kNumH : kNumF; }
// A tile survives if its LDS fits and its kernel compiles without spilling
// (measured with hipcc for gfx950: the fp32 head-dim-128 kernel with 8 waves
// spills; the build fails on any other kernel that uses scratch memory).
constexpr bool tile_ok(int dt, int D, int i) {
  return lds_bytes(dt == 0 ? 2 : 4, D, tile_at(dt, i).bn, tile_at(dt, i).nb) <= kLdsMax &&
         !(dt == 1 && D == 128 && tile_at(dt, i).nw == 8);
}
// Map compact id (among fitting tiles) -> raw index, or -1.
constexpr int raw_index(int dt, int D, int id) {
  int n = 0;
  for (int i = 0; i < num_tiles_raw(dt); ++i) {
    if (tile_ok(dt, D, i)) {
      if (n == id) return i;
      ++n;
    }
  }
  return -1;
}
constexpr int count_ok(int dt, int D) {
  int n = 0;
  for (int i = 0; i < num_tiles_raw(dt); ++i) n += tile_ok(dt, D, i) ? 1 : 0;
  return n;
}

template <class T, int D, int BN, int NW, int NB, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdArgs a) {
  typedef Mfma<T> M;
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int LS = LdsRow<T, D>::LS;
  constexpr int NKS = D / M::KSTEP;      // k-steps over the head dim
  constexpr int NDB = (D + 31) / 32;     // 32-row blocks of O^T
  constexpr int NKB = BN / 32;           // 32-key blocks per tile
  constexpr int TPB = 32 / M::KSTEP;     // k-steps per 32-key block in P V
  __shared__ __attribute__((aligned(16))) T Ks[NB][BN * LS];
  __shared__ __attribute__((aligned(16))) T Vs[NB][BN * LS];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);  // a head's blocks on one XCD (its L2 holds their K/V)
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int b = bh / a.H, h = bh % a.H;

  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  T* obase = (T*)a.o.p + b * a.o.sb + h * a.o.sh;

  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;

  typename M::frag qf[NKS];
  load_row_frags<T, D>(qf, qbase, a.q.ss, a.q.sd, qi, a.Sq, a.vec & VEC_Q);

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  const bool veck = a.vec & VEC_K, vecv = a.vec & VEC_V;

  // One tile's scores, online-softmax update and O += P V, from LDS.
  auto compute = [&](const T* Kt, const T* Vt, int k0) {
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = dot_block<T, D, LS>(Kt, kb * 32, qf);
    const bool need_mask = (k0 + BN > a.Sk) || (CAUSAL && k0 + BN - 1 > qw + a.coff);
    if (need_mask) {
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
    // m is the running row max of the raw scores q.k (before scaling).
    const float mnew = fmaxf(m, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2((m - muse) * cs);
    const float mc = muse * cs;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // fp16: one FMA per score.  fp32: subtract first, so that the rounding
        // of scale*log2(e) only scales the small difference s - max.
        float p;
        if constexpr (sizeof(T) == 2)
          p = fast_exp2(__builtin_fmaf(s[kb][r], cs, -mc));
        else
          p = fast_exp2((s[kb][r] - muse) * cs);
        s[kb][r] = p;
        rs += p;
      }
    lsum = lsum * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const typename M::frag pf = frag_from_acc<T>(s[kb], tt);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = M::mma(frag_tr<T, LS>(Vt, kb * 32, tt, db * 32), pf, oacc[db]);
      }
  };

  if constexpr (NB == 1) {
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = t * BN;
      __syncthreads();
      load_tile<T, BN, D, LS, NT>(Ks[0], kbase, a.k.ss, a.k.sd, k0, a.Sk, veck);
      load_tile<T, BN, D, LS, NT>(Vs[0], vbase, a.v.ss, a.v.sd, k0, a.Sk, vecv);
      __syncthreads();
      if (CAUSAL && k0 > qw + a.coff + 31) continue;  // every key of the tile is after every row of this wave
      compute(Ks[0], Vs[0], k0);
    }
  } else {
    TileStage<T, BN, D, LS, NT> sk, sv;
    if (ntiles > 0) {
      sk.load(kbase, a.k.ss, a.k.sd, 0, a.Sk, veck);
      sv.load(vbase, a.v.ss, a.v.sd, 0, a.Sk, vecv);
      sk.store(Ks[0]);
      sv.store(Vs[0]);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = t * BN, cur = t & 1;
      const bool more = t + 1 < ntiles;
      if (more) {
        sk.load(kbase, a.k.ss, a.k.sd, k0 + BN, a.Sk, veck);
        sv.load(vbase, a.v.ss, a.v.sd, k0 + BN, a.Sk, vecv);
      }
      // A wave whose rows all precede the tile still stages and syncs.
      if (!(CAUSAL && k0 > qw + a.coff + 31)) compute(Ks[cur], Vs[cur], k0);
      if (more) {  // the other buffer was last read before the previous barrier
        sk.store(Ks[cur ^ 1]);
        sv.store(Vs[cur ^ 1]);
      }
      __syncthreads();
    }
  }

  const float ltot = lsum + xor32(lsum);
  if (qi < a.Sq) {
    // A row with no visible key (bottom-right alignment, Sq > Sk) has
    // ltot = 0: O = 0 and LSE = -inf.
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    T* orow = obase + (int64_t)qi * a.o.ss;
    const bool veco = a.vec & VEC_O;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = oacc[db][r4 * 4 + e] * inv;
        store4<T, D>(orow, a.o.sd, db * 32 + r4 * 8 + g * 4, v4, veco);
      }
    if (g == 0)
      a.lse[(int64_t)bh * a.Sq + qi] =
          ltot > 0.f ? __builtin_fmaf(a.scale, m, fast_log2(ltot) * kLn2) : -INFINITY;
  }
}

template <class T, int D, int I, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
  constexpr int dt = sizeof(T) == 2 ? 0 : 1;
  constexpr FwdTile tl = tile_at(dt, I);
  constexpr int BM = 32 * tl.nw;
  const int64_t nqb = ((int64_t)a.Sq + BM - 1) / BM;
  const int64_t grid = nqb * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<T, D, tl.bn, tl.nw, tl.nb, CAUSAL>), dim3((unsigned)grid), dim3(tl.nw * 64), args, 0, s);
}

template <class T, int D, int I = 0>
hipError_t dispatch(const FwdArgs& a, int raw, int causal, hipStream_t s) {
  constexpr int dt = sizeof(T) == 2 ? 0 : 1;
  if constexpr (I >= num_tiles_raw(dt)) {
    return hipErrorInvalidValue;
  } else {
    if (raw == I) {
      if constexpr (tile_ok(dt, D, I)) {
        return causal ? launch_one<T, D, I, true>(a, s) : launch_one<T, D, I, false>(a, s);
      } else {
        return hipErrorInvalidValue;
      }
    }
    return dispatch<T, D, I + 1>(a, raw, causal, s);
  }
}

constexpr int count_for(int dt, int D) { return count_ok(dt, D); }

}  // namespace

// 16-bit types with head dim 128 or 64 put the tuned kernel's variants
// (fa_fwd_f16.hip) first in their tables; the generic entries follow.
static int fast_count(int dtype, int D) { return table_dt(dtype) == 0 ? fwd_fast_variants(D) : 0; }

static int generic_count(int dtype, int D) {
  switch (D) {
    case 16: return count_for(table_dt(dtype), 16);
    case 32: return count_for(table_dt(dtype), 32);
    case 64: return count_for(table_dt(dtype), 64);
    case 128: return count_for(table_dt(dtype), 128);
  }
  return 0;
}

int fwd_tile_count(int dtype, int D) { return fast_count(dtype, D) + generic_count(dtype, D); }

static int raw_for(int dtype, int D, int id) {
  switch (D) {
    case 16: return raw_index(table_dt(dtype), 16, id);
    case 32: return raw_index(table_dt(dtype), 32, id);
    case 64: return raw_index(table_dt(dtype), 64, id);
    case 128: return raw_index(table_dt(dtype), 128, id);
  }
  return -1;
}

const TileCfg* fwd_tile(int dtype, int D, int id) {
  static thread_local TileCfg cfg;
  if (id < 0 || id >= fwd_tile_count(dtype, D)) return nullptr;
  const int nf = fast_count(dtype, D);
  if (id < nf) {
    cfg = fwd_fast_cfg(id, D);
    return &cfg;
  }
  const int raw = raw_for(dtype, D, id - nf);
  const FwdTile t = tile_at(table_dt(dtype), raw);
  cfg = TileCfg{32 * t.nw, t.bn, t.nw, lds_bytes(elem_size(dtype), D, t.bn, t.nb)};
  return &cfg;
}

int fwd_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal) {
  // 16-bit, D = 128, by measurement on MI355X: the pipelined 8-wave kernel
  // with buffer loads into LDS from causal S = 2048 and non-causal S = 1024
  // up (8-15 % over the register-staged pipelined kernel); for shorter
  // sequences the plain 4-wave kernel (twice the workgroups, two per CU),
  // 1-14 % faster there.
  (void)Sq;
  if (table_dt(dtype) == 0 && D == 128) return (causal ? Sk <= 1024 : Sk <= 512) ? 3 : 4;
  return 0;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s) {
  const int nf = fast_count(dtype, D);
  if (tile < nf) {
    // The tuned kernel needs 16-byte vector access to q, k, v and out (and,
    // at D = 64, 31-bit row offsets); other arguments run the generic
    // kernel's first entry instead.
    const int need = VEC_Q | VEC_K | VEC_V | VEC_O;
    if ((a.vec & need) == need && fwd_fast_runs(a, dtype, D))
      return launch_fwd_fast(a, tile, dtype, D, causal, s);
    tile = nf;
  }
  const int raw = raw_for(dtype, D, tile - nf);
  if (raw < 0) return hipErrorInvalidValue;
  if (dtype == 0) {
    switch (D) {
      case 16: return dispatch<half_t, 16>(a, raw, causal, s);
      case 32: return dispatch<half_t, 32>(a, raw, causal, s);
      case 64: return dispatch<half_t, 64>(a, raw, causal, s);
      case 128: return dispatch<half_t, 128>(a, raw, causal, s);
    }
  } else if (dtype == 2) {
    switch (D) {
      case 16: return dispatch<bf16_t, 16>(a, raw, causal, s);
      case 32: return dispatch<bf16_t, 32>(a, raw, causal, s);
      case 64: return dispatch<bf16_t, 64>(a, raw, causal, s);
      case 128: return dispatch<bf16_t, 128>(a, raw, causal, s);
    }
  } else {
    switch (D) {
      case 16: return dispatch<float, 16>(a, raw, causal, s);
      case 32: return dispatch<float, 32>(a, raw, causal, s);
      case 64: return dispatch<float, 64>(a, raw, causal, s);
      case 128: return dispatch<float, 128>(a, raw, causal, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
