// Backward dK/dV kernel for gfx950, and the rowsum(dO.O) preprocess.
//
// Method: "Triton FlashAttention", opening summary (a backward with no
// atomics: key-side gradients and query-side gradients are produced by two
// separate kernels, each recomputing the probabilities from the forward's
// saved log-sum-exp, after a small kernel that forms the per-row dot product
// of dO with O); "FlashAttention-2 from PyTorch to Triton", backward outline
// (each key tile visits every query tile, using L and that per-row dot
// product).
//
// One workgroup owns BN = 32*waves keys of one (batch, head); each wave keeps
// its 32 keys' K and V fragments in registers and accumulates dK^T and dV^T
// (fp32) while query tiles of BM rows (Q, dO, LSE, delta) stream through LDS.
// Per 32-query block:
//   S  = Q K^T            (C layout: lane = key, registers = queries)
//   P  = exp2(S*scale*log2e - LSE*log2e)
//   dV^T += dO^T P        (dO^T read transposed from LDS)
//   dP = dO V^T
//   dS = P o (dP - delta)
//   dK^T += Q^T dS        (Q^T read transposed from LDS)
// and dK is scaled by `scale` on the way out.  Each output row is written by
// exactly one workgroup.
#include "fa_args.h"
#include "fa_common.h"

namespace fa {

namespace {

constexpr int kLdsMax = 65536;

// ----------------------------------------------------------------- preprocess
// delta[bh, i] = sum_d dO[i, d] * O[i, d] in fp32.  G threads share a row,
// each reading 16-byte chunks; a workgroup covers NP*256/G consecutive rows
// of one (batch, head), all of whose loads are issued before any is summed.
constexpr int kPrePasses = 4;

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int CH = 16 / (int)sizeof(T);
  constexpr int G = D / CH;  // threads per row (power of two, <= 32)
  constexpr int RPP = 256 / G, NP = kPrePasses;
  const int nblk = (a.Sq + RPP * NP - 1) / (RPP * NP);
  const int bh = (int)blockIdx.x / nblk;
  const int blk = (int)blockIdx.x - bh * nblk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int part = threadIdx.x % G, col = part * CH;
  const T* obase = (const T*)a.o.p + b * a.o.sb + h * a.o.sh;
  const T* dbase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  T ov[NP][CH], dv[NP][CH];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int i = min((blk * NP + p) * RPP + (int)threadIdx.x / G, a.Sq - 1);  // tail rows clamped
    const T* orow = obase + (int64_t)i * a.o.ss;
    const T* drow = dbase + (int64_t)i * a.dout.ss;
    if (a.vec & VEC_O) {
      const uint4 x = *reinterpret_cast<const uint4*>(orow + col);  // 16-byte aligned (checked on the host)
      __builtin_memcpy(ov[p], &x, 16);
    } else {
#pragma unroll
      for (int e = 0; e < CH; ++e) ov[p][e] = orow[(int64_t)(col + e) * a.o.sd];
    }
    if (a.vec & VEC_DO) {
      const uint4 x = *reinterpret_cast<const uint4*>(drow + col);  // 16-byte aligned (checked on the host)
      __builtin_memcpy(dv[p], &x, 16);
    } else {
#pragma unroll
      for (int e = 0; e < CH; ++e) dv[p][e] = drow[(int64_t)(col + e) * a.dout.sd];
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc = __builtin_fmaf((float)dv[p][e], (float)ov[p][e], acc);
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    const int i = (blk * NP + p) * RPP + (int)threadIdx.x / G;
    if (i < a.Sq && part == 0) a.delta[(int64_t)bh * a.Sq + i] = acc;
  }
}

// ----------------------------------------------------------------- dK / dV
// Query rows per tile, waves, and Q/dO buffers in LDS (1: load then compute,
// two barriers per tile; 2: the next tile's global reads are issued into
// registers before the current tile is computed and stored to the other
// buffer after it, one barrier per tile).  New configurations go at the end
// so that the ids of the existing ones do not move.
struct Tile { int bm, nw, nb; };
constexpr Tile kTilesH[] = {{64, 4, 1}, {32, 4, 1}, {64, 2, 1}, {128, 4, 1}, {32, 8, 1},
                            {64, 4, 2}, {32, 4, 2}, {64, 2, 2}};
constexpr Tile kTilesF[] = {{32, 4, 1}, {32, 2, 1}, {64, 4, 1}, {32, 4, 2}, {32, 2, 2}};
constexpr int kNumH = sizeof(kTilesH) / sizeof(kTilesH[0]);
constexpr int kNumF = sizeof(kTilesF) / sizeof(kTilesF[0]);

constexpr int lds_bytes(int esize, int D, int bm, int nb) {
  return nb * (2 * bm * ((D < 32 ? 32 : D) + 16 / esize) * esize + 2 * bm * 4);
}
constexpr Tile tile_at(int dt, int i) { return dt == 0 ? kTilesH[i] : kTilesF[i]; }
constexpr int num_tiles_raw(int dt) { return dt == 0 ? kNumH : kNumF; }
// A tile survives if its LDS fits and its kernel compiles without spilling
// (measured with hipcc for gfx950: at head dim 128 the 16-bit 8-wave kernel
// spills, and so does the fp32 2-wave one; the build fails on any kernel that
// uses scratch memory).
constexpr bool tile_ok(int dt, int D, int i) {
  return lds_bytes(dt == 0 ? 2 : 4, D, tile_at(dt, i).bm, tile_at(dt, i).nb) <= kLdsMax &&
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

template <class T, int D, int BM, int NW, int NB, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(BwdArgs a) {
  typedef Mfma<T> M;
  constexpr int BN = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int LS = LdsRow<T, D>::LS;
  constexpr int NKS = D / M::KSTEP;
  // fp32 at head dim 128: K and V fragments (128 registers) and the dK, dV
  // accumulators of all four 32-column blocks (256) do not fit one wave, so
  // the kernel runs twice over the queries, accumulating two column blocks
  // of dK and dV each time (the scores are recomputed).
  constexpr int NPASS = (sizeof(T) == 4 && D == 128) ? 2 : 1;
  constexpr int NDB = (D + 31) / 32 / NPASS;  // 32-column blocks per pass
  constexpr int NQB = BM / 32;
  constexpr int TPB = 32 / M::KSTEP;
  __shared__ __attribute__((aligned(16))) T Qs[NB][BM * LS];
  __shared__ __attribute__((aligned(16))) T Ds[NB][BM * LS];
  __shared__ float Ls[NB][BM];
  __shared__ float Dl[NB][BM];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, c = lane & 31;
  const int nkb = (a.Sk + BN - 1) / BN;
  int kb, bh;
  xcd_block(nkb, CAUSAL, kb, bh);  // a head's blocks on one XCD; causal key block 0 (the longest) first
  const int b = bh / a.H, h = bh % a.H;
  const int k0 = kb * BN, kw = k0 + w * 32, kj = kw + c;

  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* kbase = (const T*)a.k.p + b * a.k.sb + h * a.k.sh;
  const T* vbase = (const T*)a.v.p + b * a.v.sb + h * a.v.sh;
  const T* dobase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  const float* lse = a.lse + (int64_t)bh * a.Sq;
  const float* dl = a.delta + (int64_t)bh * a.Sq;

  typename M::frag kf[NKS], vf[NKS];
  load_row_frags<T, D>(kf, kbase, a.k.ss, a.k.sd, kj, a.Sk, a.vec & VEC_K);
  load_row_frags<T, D>(vf, vbase, a.v.ss, a.v.sd, kj, a.Sk, a.vec & VEC_V);
  if constexpr (NPASS == 2) {
    // fp32 at head dim 128: K and V (128 registers) stay in accumulator
    // registers as MFMA operands (this file is built with the VGPR
    // accumulator form), leaving the architectural file to the scores and
    // the dK, dV sums.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      asm("" : "+a"(kf[ks]));
      asm("" : "+a"(vf[ks]));
    }
  }

  f32x16 dk[NDB], dv[NDB];
  const float cs = a.scale_log2;
  const bool vecq = a.vec & VEC_Q, vecd = a.vec & VEC_DO;
  const bool key_tail = k0 + BN > a.Sk;
  int d0 = 0;  // first column of this pass's blocks

  // LSE (fp16 kernels: LSE*log2(e); fp32 kernels: LSE itself) and delta of
  // tile row r.  Rows past the end, and rows with no visible key (LSE =
  // -inf), get P = 0.
  auto row_ls = [&](int i) {
    const float li = i < a.Sq ? lse[i] : INFINITY;
    return li == -INFINITY ? INFINITY : (sizeof(T) == 2 ? li * kLog2e : li);
  };
  auto row_dl = [&](int i) { return i < a.Sq ? dl[i] : 0.f; };

  // One tile of BM query rows starting at q0, from LDS.
  auto compute = [&](const T* Qt, const T* Dt, const float* Lt, const float* Mt, int q0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qs = q0 + qb * 32;
      if (CAUSAL && qs + a.coff + 31 < kw) continue;  // every query of the block precedes every key
      f32x16 s = dot_block<T, D, LS>(Qt, qb * 32, kf);
      const bool need_mask = key_tail || (CAUSAL && qs + a.coff < kw + 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = qb * 32 + crow(r, g);
        float p;
        if constexpr (sizeof(T) == 2)
          p = fast_exp2(__builtin_fmaf(s[r], cs, -Lt[qr]));
        else
          p = fast_exp2(__builtin_fmaf(a.scale, s[r], -Lt[qr]) * kLog2e);
        if (need_mask && (kj >= a.Sk || (CAUSAL && kj > q0 + qr + a.coff))) p = 0.f;
        s[r] = p;
      }
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const typename M::frag pf = frag_from_acc<T>(s, tt);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dv[db] = M::mma(frag_tr<T, LS>(Dt, qb * 32, tt, d0 + db * 32), pf, dv[db]);
      }
      const f32x16 dp = dot_block<T, D, LS>(Dt, qb * 32, vf);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = qb * 32 + crow(r, g);
        s[r] = s[r] * (dp[r] - Mt[qr]);
      }
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const typename M::frag df = frag_from_acc<T>(s, tt);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dk[db] = M::mma(frag_tr<T, LS>(Qt, qb * 32, tt, d0 + db * 32), df, dk[db]);
      }
    }
  };

  const int qstart = CAUSAL ? (max(0, k0 - a.coff) / BM) * BM : 0;
  T* dkrow = (T*)a.dk.p + b * a.dk.sb + h * a.dk.sh + (int64_t)kj * a.dk.ss;
  T* dvrow = (T*)a.dv.p + b * a.dv.sb + h * a.dv.sh + (int64_t)kj * a.dv.ss;
  const bool veck = a.vec & VEC_DK, vecv = a.vec & VEC_DV;
  for (int pass = 0; pass < NPASS; ++pass) {
  d0 = pass * NDB * 32;
#pragma unroll
  for (int i = 0; i < NDB; ++i) { dk[i] = zero16(); dv[i] = zero16(); }
  if (pass > 0) __syncthreads();  // the previous pass's last tile has been read
  if constexpr (NB == 1) {
    for (int q0 = qstart; q0 < a.Sq; q0 += BM) {
      __syncthreads();
      load_tile<T, BM, D, LS, NT>(Qs[0], qbase, a.q.ss, a.q.sd, q0, a.Sq, vecq);
      load_tile<T, BM, D, LS, NT>(Ds[0], dobase, a.dout.ss, a.dout.sd, q0, a.Sq, vecd);
      for (int r = threadIdx.x; r < BM; r += NT) {
        Ls[0][r] = row_ls(q0 + r);
        Dl[0][r] = row_dl(q0 + r);
      }
      __syncthreads();
      compute(Qs[0], Ds[0], Ls[0], Dl[0], q0);
    }
  } else {
    static_assert(BM <= NT, "one thread per staged LSE / delta row");
    TileStage<T, BM, D, LS, NT> sq, sd;
    float rl = 0.f, rd = 0.f;
    const int r = threadIdx.x;
    auto stage = [&](int q0) {
      sq.load(qbase, a.q.ss, a.q.sd, q0, a.Sq, vecq);
      sd.load(dobase, a.dout.ss, a.dout.sd, q0, a.Sq, vecd);
      if (r < BM) {
        rl = row_ls(q0 + r);
        rd = row_dl(q0 + r);
      }
    };
    auto put = [&](int buf) {
      sq.store(Qs[buf]);
      sd.store(Ds[buf]);
      if (r < BM) {
        Ls[buf][r] = rl;
        Dl[buf][r] = rd;
      }
    };
    const int ntiles = a.Sq > qstart ? (a.Sq - qstart + BM - 1) / BM : 0;
    if (ntiles > 0) {
      stage(qstart);
      put(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int q0 = qstart + t * BM, cur = t & 1;
      const bool more = t + 1 < ntiles;
      if (more) stage(q0 + BM);
      compute(Qs[cur], Ds[cur], Ls[cur], Dl[cur], q0);
      if (more) put(cur ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }

  if (kj < a.Sk) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float k4[4], v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = dk[db][r4 * 4 + e] * a.scale;
          v4[e] = dv[db][r4 * 4 + e];
        }
        store4<T, D>(dkrow, a.dk.sd, d0 + db * 32 + r4 * 8 + g * 4, k4, veck);
        store4<T, D>(dvrow, a.dv.sd, d0 + db * 32 + r4 * 8 + g * 4, v4, vecv);
      }
  }
  }  // pass
}

template <class T, int D, int I, bool CAUSAL>
hipError_t launch_one(const BwdArgs& a, hipStream_t s) {
  constexpr int dt = sizeof(T) == 2 ? 0 : 1;
  constexpr Tile tl = tile_at(dt, I);
  constexpr int BN = 32 * tl.nw;
  const int64_t nkb = ((int64_t)a.Sk + BN - 1) / BN;
  const int64_t grid = nkb * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dkdv_kernel<T, D, tl.bm, tl.nw, tl.nb, CAUSAL>), dim3((unsigned)grid), dim3(tl.nw * 64), args, 0, s);
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

template <class T, int D>
hipError_t launch_pre_t(const BwdArgs& a, hipStream_t s) {
  constexpr int G = D / (16 / (int)sizeof(T));
  constexpr int RPB = 256 / G * kPrePasses;
  const int64_t grid = (((int64_t)a.Sq + RPB - 1) / RPB) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<T, D>), dim3((unsigned)grid), dim3(256), args, 0, s);
}

}  // namespace

// 16-bit types with head dim 128 or 64 put the tuned kernel's variants
// (fa_bwd_f16.hip) first in their tables; the generic entries follow.
static int fast_count(int dtype, int D) { return table_dt(dtype) == 0 ? dkdv_fast_variants(D) : 0; }

static int generic_count(int dtype, int D) {
  switch (D) {
    case 16: return count_ok(table_dt(dtype), 16);
    case 32: return count_ok(table_dt(dtype), 32);
    case 64: return count_ok(table_dt(dtype), 64);
    case 128: return count_ok(table_dt(dtype), 128);
  }
  return 0;
}

int dkdv_tile_count(int dtype, int D) { return fast_count(dtype, D) + generic_count(dtype, D); }

const TileCfg* dkdv_tile(int dtype, int D, int id) {
  static thread_local TileCfg cfg;
  if (id < 0 || id >= dkdv_tile_count(dtype, D)) return nullptr;
  const int nf = fast_count(dtype, D);
  if (id < nf) {
    cfg = dkdv_fast_cfg(id, D);
    return &cfg;
  }
  id -= nf;
  const Tile t = tile_at(table_dt(dtype), raw_for(dtype, D, id));
  cfg = TileCfg{t.bm, 32 * t.nw, t.nw, lds_bytes(elem_size(dtype), D, t.bm, t.nb)};
  return &cfg;
}

int dkdv_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal) {
  (void)Sq; (void)Sk; (void)causal;
  // 16-bit, D = 128: the software-pipelined tuned kernel (128-query tiles,
  // swizzled single-copy layout, buffer loads into LDS) measured fastest on
  // MI355X at every length from 512 to 16384, causal and not.
  if (table_dt(dtype) == 0 && D == 128) return 4;
  // 16-bit, D = 64: the same kernel with two waves per SIMD, fastest at every
  // length from 128 to 16384.
  if (table_dt(dtype) == 0 && D == 64) return 1;
  return 0;
}

hipError_t launch_dkdv(const BwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s) {
  const int nf = fast_count(dtype, D);
  if (tile < nf) {
    // The tuned kernel needs 16-byte vector access to every tensor it touches
    // (and, at D = 64, 31-bit row offsets); other arguments run the generic
    // kernel's first entry instead.
    const int need = VEC_Q | VEC_K | VEC_V | VEC_DO | VEC_DK | VEC_DV;
    if ((a.vec & need) == need && dkdv_fast_runs(a, dtype, D))
      return launch_dkdv_fast(a, tile, dtype, D, causal, s);
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

hipError_t launch_bwd_pre(const BwdArgs& a, int dtype, int D, hipStream_t s) {
  if (dtype == 0) {
    switch (D) {
      case 16: return launch_pre_t<half_t, 16>(a, s);
      case 32: return launch_pre_t<half_t, 32>(a, s);
      case 64: return launch_pre_t<half_t, 64>(a, s);
      case 128: return launch_pre_t<half_t, 128>(a, s);
    }
  } else if (dtype == 2) {
    switch (D) {
      case 16: return launch_pre_t<bf16_t, 16>(a, s);
      case 32: return launch_pre_t<bf16_t, 32>(a, s);
      case 64: return launch_pre_t<bf16_t, 64>(a, s);
      case 128: return launch_pre_t<bf16_t, 128>(a, s);
    }
  } else {
    switch (D) {
      case 16: return launch_pre_t<float, 16>(a, s);
      case 32: return launch_pre_t<float, 32>(a, s);
      case 64: return launch_pre_t<float, 64>(a, s);
      case 128: return launch_pre_t<float, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
