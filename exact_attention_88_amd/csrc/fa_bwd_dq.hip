// Backward dQ kernel for gfx950.
//
// Method: "Triton FlashAttention", opening summary (the query-side half of
// the atomic-free backward).  Each workgroup owns a block of query rows and
// visits the key tiles it can see, so every dQ row has exactly one writer;
// the probabilities are recomputed from the saved log-sum-exp.
//
// One workgroup owns BM = 32*waves query rows of one (batch, head); each wave
// keeps its 32 rows' Q and dO fragments, LSE and delta in registers and
// accumulates dQ^T (fp32) while K and V tiles of BN keys stream through LDS.
// Per 32-key block, computed transposed so that each lane owns one query:
//   S^T  = K Q^T
//   P^T  = exp2(S^T*scale*log2e - LSE*log2e)
//   dP^T = V dO^T
//   dS^T = P^T o (dP^T - delta)
//   dQ^T += K^T dS^T      (K^T read transposed from LDS)
// and dQ is scaled by `scale` on the way out.
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
struct Tile { int bn, nw, nb; };
constexpr Tile kTilesH[] = {{64, 4, 1}, {32, 4, 1}, {64, 2, 1}, {128, 4, 1}, {64, 8, 1},
                            {64, 4, 2}, {32, 4, 2}, {64, 8, 2}};
constexpr Tile kTilesF[] = {{32, 4, 1}, {32, 2, 1}, {64, 4, 1}, {32, 4, 2}};
constexpr int kNumH = sizeof(kTilesH) / sizeof(kTilesH[0]);
constexpr int kNumF = sizeof(kTilesF) / sizeof(kTilesF[0]);

constexpr int lds_bytes(int esize, int D, int bn, int nb) {
  return nb * 2 * bn * ((D < 32 ? 32 : D) + 16 / esize) * esize;
}
constexpr Tile tile_at(int dt, int i) { return dt == 0 ? kTilesH[i] : kTilesF[i]; }
constexpr int num_tiles_raw(int dt) { return dt == 0 ? kNumH : kNumF; }
// A tile survives if its LDS fits and its kernel compiles without spilling
// (measured with hipcc for gfx950: at head dim 128 the 16-bit 8-wave kernel
// spills, and so does the fp32 2-wave one; the fp32 4-wave one spills a
// little when non-causal and is kept, so that fp32 D = 128 has a kernel.  The
// build fails on any other kernel that uses scratch memory).
constexpr bool tile_ok(int dt, int D, int i) {
  return lds_bytes(dt == 0 ? 2 : 4, D, tile_at(dt, i).bn, tile_at(dt, i).nb) <= kLdsMax &&
         !(D == 128 && dt == 0 && tile_at(dt, i).nw == 8) &&
         !(D == 128 && dt == 1 && tile_at(dt, i).nw == 2);
}
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
__global__ __launch_bounds__(NW * 64) void dq_kernel(BwdArgs a) {
  typedef Mfma<T> M;
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int LS = LdsRow<T, D>::LS;
  constexpr int NKS = D / M::KSTEP;
  constexpr int NDB = (D + 31) / 32;
  constexpr int NKB = BN / 32;
  constexpr int TPB = 32 / M::KSTEP;
  __shared__ __attribute__((aligned(16))) T Ks[NB][BN * LS];
  __shared__ __attribute__((aligned(16))) T Vs[NB][BN * LS];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nqb = (a.Sq + BM - 1) / BM;
  int qb, bh;
  xcd_block(nqb, CAUSAL, qb, bh);  // a head's blocks on one XCD (its L2 holds their K/V)
  if (CAUSAL) qb = nqb - 1 - qb;    // longest rows first
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * BM, qw = q0 + w * 32, qi = qw + c;

  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  const T* dobase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;

  typename M::frag qf[NKS], df[NKS];
  load_row_frags<T, D>(qf, qbase, a.q.ss, a.q.sd, qi, a.Sq, a.vec & VEC_Q);
  load_row_frags<T, D>(df, dobase, a.dout.ss, a.dout.sd, qi, a.Sq, a.vec & VEC_DO);
  const bool valid = qi < a.Sq;
  // fp16 uses LSE*log2(e) in one FMA per score; fp32 uses LSE itself (see below).
  // Rows past the end, and rows with no visible key (LSE = -inf), get P = 0.
  float lse_n = valid ? a.lse[(int64_t)bh * a.Sq + qi] : INFINITY;
  if (lse_n == -INFINITY) lse_n = INFINITY;
  const float lse2 = sizeof(T) == 2 ? lse_n * kLog2e : lse_n;
  const float dlt = valid ? a.delta[(int64_t)bh * a.Sq + qi] : 0.f;

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = zero16();
  const float cs = a.scale_log2;
  const bool veck = a.vec & VEC_K, vecv = a.vec & VEC_V;

  const int kend = CAUSAL ? max(0, min(a.Sk, q0 + a.coff + BM)) : a.Sk;
  const int ntiles = (kend + BN - 1) / BN;
  // One tile: per 32-key block, P, dS and dQ += dS K, from LDS.
  auto compute = [&](const T* Kt, const T* Vt, int k0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int ks0 = k0 + kb * 32;
      if (CAUSAL && ks0 > qw + a.coff + 31) continue;  // block entirely after this wave's rows
      f32x16 s = dot_block<T, D, LS>(Kt, kb * 32, qf);
      const bool need_mask = (ks0 + 32 > a.Sk) || (CAUSAL && ks0 + 31 > qw + a.coff);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = ks0 + crow(r, g);
        float p;
        if constexpr (sizeof(T) == 2)
          p = fast_exp2(__builtin_fmaf(s[r], cs, -lse2));
        else
          p = fast_exp2(__builtin_fmaf(a.scale, s[r], -lse2) * kLog2e);
        if (need_mask && (key >= a.Sk || (CAUSAL && key > qi + a.coff))) p = 0.f;
        s[r] = p;
      }
      const f32x16 dp = dot_block<T, D, LS>(Vt, kb * 32, df);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - dlt);
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const typename M::frag sf = frag_from_acc<T>(s, tt);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dq[db] = M::mma(frag_tr<T, LS>(Kt, kb * 32, tt, db * 32), sf, dq[db]);
      }
    }
  };
  if constexpr (NB == 1) {
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = t * BN;
      __syncthreads();
      load_tile<T, BN, D, LS, NT>(Ks[0], kbase, a.k.ss, a.k.sd, k0, a.Sk, veck);
      load_tile<T, BN, D, LS, NT>(Vs[0], vbase, a.v.ss, a.v.sd, k0, a.Sk, vecv);
      __syncthreads();
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
      compute(Ks[cur], Vs[cur], k0);
      if (more) {  // the other buffer was last read before the previous barrier
        sk.store(Ks[cur ^ 1]);
        sv.store(Vs[cur ^ 1]);
      }
      __syncthreads();
    }
  }

  if (valid) {
    T* row = (T*)a.dq.p + b * a.dq.sb + h * a.dq.sh + (int64_t)qi * a.dq.ss;
    const bool vecq = a.vec & VEC_DQ;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = dq[db][r4 * 4 + e] * a.scale;
        store4<T, D>(row, a.dq.sd, db * 32 + r4 * 8 + g * 4, v4, vecq);
      }
  }
}

template <class T, int D, int I, bool CAUSAL>
hipError_t launch_one(const BwdArgs& a, hipStream_t s) {
  constexpr int dt = sizeof(T) == 2 ? 0 : 1;
  constexpr Tile tl = tile_at(dt, I);
  constexpr int BM = 32 * tl.nw;
  const int64_t nqb = ((int64_t)a.Sq + BM - 1) / BM;
  const int64_t grid = nqb * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dq_kernel<T, D, tl.bn, tl.nw, tl.nb, CAUSAL>), dim3((unsigned)grid), dim3(tl.nw * 64), args, 0, s);
}

template <class T, int D, int I = 0>
hipError_t dispatch(const BwdArgs& a, int raw, int causal, hipStream_t s) {
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

int raw_for(int dtype, int D, int id) {
  switch (D) {
    case 16: return raw_index(table_dt(dtype), 16, id);
    case 32: return raw_index(table_dt(dtype), 32, id);
    case 64: return raw_index(table_dt(dtype), 64, id);
    case 128: return raw_index(table_dt(dtype), 128, id);
  }
  return -1;
}

}  // namespace

// 16-bit types with head dim 128 or 64 put the tuned kernel's variants
// (fa_bwd_f16.hip) first in their tables; the generic entries follow.
static int fast_count(int dtype, int D) { return table_dt(dtype) == 0 ? dq_fast_variants(D) : 0; }

static int generic_count(int dtype, int D) {
  switch (D) {
    case 16: return count_ok(table_dt(dtype), 16);
    case 32: return count_ok(table_dt(dtype), 32);
    case 64: return count_ok(table_dt(dtype), 64);
    case 128: return count_ok(table_dt(dtype), 128);
  }
  return 0;
}

int dq_tile_count(int dtype, int D) { return fast_count(dtype, D) + generic_count(dtype, D); }

const TileCfg* dq_tile(int dtype, int D, int id) {
  static thread_local TileCfg cfg;
  if (id < 0 || id >= dq_tile_count(dtype, D)) return nullptr;
  const int nf = fast_count(dtype, D);
  if (id < nf) {
    cfg = dq_fast_cfg(id, D);
    return &cfg;
  }
  id -= nf;
  const Tile t = tile_at(table_dt(dtype), raw_for(dtype, D, id));
  cfg = TileCfg{32 * t.nw, t.bn, t.nw, lds_bytes(elem_size(dtype), D, t.bn, t.nb)};
  return &cfg;
}

int dq_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal) {
  (void)Sq; (void)Sk; (void)causal;
  // 16-bit, D = 128: the tuned kernel with 8 waves, 64-key tiles in the
  // swizzled single-copy layout and buffer loads into LDS measured fastest on
  // MI355X at S = 4096 and 16384, causal and not.
  if (table_dt(dtype) == 0 && D == 128) return 5;
  // 16-bit, D = 64: the buffer-load kernel with 4 waves, fastest at every
  // length from 128 to 16384.
  if (table_dt(dtype) == 0 && D == 64) return 1;
  return 0;
}

bool dq_can_fuse_delta(const BwdArgs& a, int dtype, int D, int tile) {
  if (tile >= fast_count(dtype, D)) return false;
  const int need = VEC_Q | VEC_K | VEC_V | VEC_DO | VEC_DQ | VEC_O;
  return (a.vec & need) == need && dq_fast_fuses_delta(a, tile, dtype, D);
}

hipError_t launch_dq(const BwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s) {
  const int nf = fast_count(dtype, D);
  if (tile < nf) {
    // The tuned kernel needs 16-byte vector access to every tensor it touches
    // (and, at D = 64, 31-bit row offsets); other arguments run the generic
    // kernel's first entry instead.
    const int need = VEC_Q | VEC_K | VEC_V | VEC_DO | VEC_DQ;
    if ((a.vec & need) == need && dq_fast_runs(a, dtype, D))
      return launch_dq_fast(a, tile, dtype, D, causal, s);
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
