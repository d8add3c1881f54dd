// Backward dK/dV kernel for 16-bit inputs (fp16, bf16) with head dim 128 on
// gfx950, with the work of each 32-key slice split between two waves.
//
// Method: "Triton FlashAttention", opening summary (key-side gradients in a
// kernel of their own, no atomics, probabilities recomputed from the saved
// log-sum-exp); "FlashAttention-2 from PyTorch to Triton", backward outline
// (each key tile visits every query tile it can see).  Per 32-query block:
//   S = Q K^T,  P = exp2(S*scale*log2e - LSE*log2e),  dV^T += dO^T P,
//   dP = dO V^T,  dS = P o (dP - delta),  dK^T += Q^T dS,
// and dK is scaled by `scale` on the way out.
//
// Layout on CDNA4.  A workgroup owns 128 keys of one (batch, head) and runs
// 8 waves, two per SIMD.  Keys are handled in four 32-key slices, each by a
// pair of waves:
//   * the score wave holds the slice's K rows and its dV accumulator; per
//     block it forms S, then P (the exponentials), hands P (fp32) to its
//     partner through LDS, and adds dO^T P to dV;
//   * the accumulate wave holds the slice's V rows and its dK accumulator;
//     per block it forms dP - delta, takes P from LDS, forms dS, and adds
//     Q^T dS to dK.
// Splitting the four accumulators (dK, dV) and the two operand sets (K, V)
// over two waves keeps each wave near 200 registers, so two waves share each
// SIMD and cover each other's LDS and exponential latency, where one wave
// holding all of them needs about 470 registers and runs alone.  The two
// waves of a pair compute every product exactly as a single wave would (same
// operands, same accumulation order, P and dS rounded the same way), so the
// results are bitwise those of the one-wave kernel.
//
// Rounds.  Blocks go through in rounds separated by one workgroup barrier.
// In round r the score wave computes P(r) from S(r) (formed in round r-1),
// publishes it, accumulates dV(r), and forms S(r+1); the accumulate wave
// forms dP(r) - delta and, from P(r-1) published in round r-1 and its own
// dP(r-1) - delta, dS(r-1) and dK(r-1).  P goes through two LDS slots
// (written in round r, read in round r+1).
//
// Tiles.  Q and dO stream in 64-query tiles (two blocks) through three LDS
// buffers, loaded straight from global memory into the XOR-swizzled layout by
// buffer loads (rows at or past Sq fall outside the buffer's byte range and
// read as zero; their LSE is stored as +inf, so P = 0 there).  Tile t is
// first read in round 2t-1 and last in round 2t+2 (the operands of the next
// round that need no barrier are read before it); tile t+3 reuses its
// buffer, is issued in round 2t+3 and is published (waited for, with its LSE
// and delta rows) at the barrier that ends round 2t+4.
//
// Measured on MI355X this kernel is 4-8 % slower than the one-wave kernel
// (dkdv_pipe_d128): the pair moves 4 KB more through LDS per 32-query round
// (P, fp32) on top of the 32 KB of Q, dO, Q^T and dO^T every 32-key slice
// reads, and both kernels are bound by LDS throughput rather than by their
// issue schedule.  It stays in the tile table as a tested alternative.
//
// Needs 31-bit byte offsets for every Q and dO row below Sq + 64 and a row
// stride of at least 128 elements (checked on the host).
#include "fa_args.h"
#include "fa_common.h"
#include "fa_lds.h"

namespace fa {

namespace {

using namespace swzl;

constexpr int kBM = 64;          // query rows per tile
constexpr int kNB = 3;           // tile buffers
constexpr int kNP = 4;           // wave pairs (key slices)
constexpr int kBN = 32 * kNP;    // keys per workgroup
constexpr int kTR = kBM * kD;    // elements of one Q or dO tile
constexpr int kXP = 16 * 64;     // floats of one pair's P block (16 per lane)

template <class T>
__device__ __forceinline__ V8<T> cvt8s(const f32x16& x, int t) {
  V8<T> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)x[t * 8 + e];
  return r;
}

template <class T>
__device__ __forceinline__ void store_rows4(T* rowp, const f32x16* acc, float mul, int g) {
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

template <class T, bool CAUSAL>
__global__ __launch_bounds__(512) void dkdv_split_d128(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) T smem[kNB * 2 * kTR];  // [buffer][Q, dO][row][d]
  __shared__ __attribute__((aligned(16))) float xp[2][kNP][kXP];      // P: [slot][pair][4][lane][4]
  __shared__ __attribute__((aligned(16))) float lsd[kNB][2][kBM];     // [buffer][LSE*log2e, -delta][row]

  const int lane = threadIdx.x & 63, g = lane >> 5, c = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool score = w < kNP;  // wave-uniform role
  const int pr = w & (kNP - 1);
  const int nkb = (a.Sk + kBN - 1) / kBN;
  int kb, bh;
  xcd_block(nkb, CAUSAL, kb, bh);
  const int b = bh / a.H, h = bh % a.H;
  const T* qbase = (const T*)a.q.p + b * a.q.sb + h * a.q.sh;
  const T* dobase = (const T*)a.dout.p + b * a.dout.sb + h * a.dout.sh;
  const rsrc_t rq = make_rsrc(qbase, (int)((int64_t)a.Sq * a.q.ss * (int64_t)sizeof(T)));
  const rsrc_t rd = make_rsrc(dobase, (int)((int64_t)a.Sq * a.dout.ss * (int64_t)sizeof(T)));
  const float* lse = a.lse + (int64_t)bh * a.Sq;
  const float* dl = a.delta + (int64_t)bh * a.Sq;
  const int k0 = kb * kBN, kw = k0 + pr * 32, kj = kw + c;

  // The slice's K rows (score waves) or V rows (accumulate waves), as the B
  // operand of S = Q K^T or dP = dO V^T: lane (c, g) holds row kj, elements
  // ks*16 + g*8 .. +7.
  V8<T> kv[8];
  {
    const int kc = min(kj, a.Sk - 1);
    const T* row = score ? (const T*)a.k.p + b * a.k.sb + h * a.k.sh + (int64_t)kc * a.k.ss
                         : (const T*)a.v.p + b * a.v.sb + h * a.v.sh + (int64_t)kc * a.v.ss;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kv[ks] = *reinterpret_cast<const V8<T>*>(row + ks * 16 + g * 8);
  }
  // K or V resident before any buffer load into LDS is issued (the compiler
  // does not count those loads).
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  const float cs = a.scale_log2;
  const int qstart = CAUSAL ? (max(0, k0 - a.coff) / kBM) * kBM : 0;
  const int nblk = a.Sq > qstart ? (a.Sq - qstart + 31) / 32 : 0;
  const int ntiles = (nblk + 1) / 2;

  const unsigned lds0 = lds_addr(smem);
  const int qsb = (int)(a.q.ss * (int64_t)sizeof(T)), dsb = (int)(a.dout.ss * (int64_t)sizeof(T));
  const int qlo = dma_lane_off<8>(qsb), dlo = dma_lane_off<8>(dsb);
  auto dma_tile = [&](int t) {
    const int q0 = qstart + t * kBM;
    const unsigned base = lds0 + (unsigned)((t % kNB) * 2 * kTR * (int)sizeof(T));
    tile_dma<kBM, 8>(rq, base, qlo, qsb, q0);
    tile_dma<kBM, 8>(rd, base + (unsigned)(kTR * (int)sizeof(T)), dlo, dsb, q0);
  };
  // LSE (in log2 units, +inf on rows past Sq or with no visible key, so that
  // P = 0 there) and -delta of one tile's rows, thread i < 64 row i.
  auto row_stats = [&](int t, int i, float& ls, float& nd) {
    const int q = qstart + t * kBM + i;
    const bool in = q < a.Sq;
    const float l = lse[min(q, a.Sq - 1)], d = dl[min(q, a.Sq - 1)];
    ls = (!in || l == -INFINITY) ? INFINITY : l * kLog2e;
    nd = in ? -d : 0.f;
  };

  // Prologue: the first three tiles (waves 0..2 fetch one tile's row
  // statistics each), published before round 0.
  {
    const int npro = min(ntiles, kNB);
    for (int t = 0; t < npro; ++t) dma_tile(t);
    float ls = 0.f, nd = 0.f;
    const int tt = (int)threadIdx.x >> 6;
    if (tt < npro) row_stats(tt, lane, ls, nd);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (tt < npro) {
      lsd[tt][0][lane] = ls;
      lsd[tt][1][lane] = nd;
    }
    __syncthreads();
  }
  // Tile t >= 3: issued at the start of round 2t-3 (all waves share the
  // loads, wave 0 fetches the row statistics), published at the barrier
  // ending round 2t-2.
  float st_ls = 0.f, st_nd = 0.f;
  auto tile_issue = [&](int r) {
    if (r >= 3 && (r & 1)) {
      const int t = (r + 3) >> 1;
      if (t < ntiles) {
        dma_tile(t);
        if (threadIdx.x < 64) row_stats(t, lane, st_ls, st_nd);
      }
    }
  };
  auto tile_publish = [&](int r) {
    if (r >= 4 && !(r & 1)) {
      const int t = (r + 2) >> 1;
      if (t < ntiles) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads are in LDS
        if (threadIdx.x < 64) {
          lsd[t % kNB][0][lane] = st_ls;
          lsd[t % kNB][1][lane] = st_nd;
        }
      }
    }
  };
  // LDS tile of block j: Q rows at qtile(j) + row offset rowoff(j), dO at + kTR.
  auto qtile = [&](int j) { return smem + ((j >> 1) % kNB) * 2 * kTR; };
  auto rowoff = [](int j) { return (j & 1) * 32; };
  auto stats = [&](int j, int which) { return &lsd[(j >> 1) % kNB][which][(j & 1) * 32]; };
  // Rows of k-step tt of an accumulator (crow order) out of four float4 runs.
  auto sel = [](const float4* v, int r) {
    return r % 4 == 0 ? v[r / 4].x : r % 4 == 1 ? v[r / 4].y : r % 4 == 2 ? v[r / 4].z : v[r / 4].w;
  };

  f32x16 acc[4];  // dV^T (score waves) or dK^T (accumulate waves): lane = key, registers = d
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();

  if (score) {
    // Block j needs the causal mask while its first query precedes the
    // slice's last key.
    const int hid = kw + 31 - a.coff - qstart;
    const int nmask = CAUSAL ? min(nblk, max(0, (hid + 31) / 32)) : 0;
    // Q rows and LSE rows of block j (operands of S(j) and P(j)).
    auto read_q = [&](int j, V8<T>* qf, float4* l4) {
      const T* Q = qtile(j);
      const int ro = rowoff(j);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = frag_r_swz(Q, ro, ks * 2);
      const float* L = stats(j, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) l4[i] = *reinterpret_cast<const float4*>(L + i * 8 + g * 4);
    };
    // dO^T of block j (operand of dV(j)).
    auto read_dt = [&](int j, V8<T> (*dt)[4]) {
      const T* D = qtile(j) + kTR;
      const int ro = rowoff(j);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db) dt[tt][db] = frag_t_swz(D, ro, tt, db * 32);
    };
    f32x16 sc;
    float4 lc[4];
    V8<T> dt[2][4];
    if (nblk > 0) {
      V8<T> qf[8];
      read_q(0, qf, lc);
      sc = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sc = Mfma<T>::mma(qf[ks], kv[ks], sc);
      read_dt(0, dt);
    }
    // Round r: P(r) from S(r) (VALU) while S(r+1) runs (MFMA), then dV(r);
    // dO^T(r+1) is read for the next round before the barrier (its tile was
    // published at least one round earlier).
    auto round = [&](auto masked, int r) {
      constexpr bool MASK = decltype(masked)::value;
      tile_issue(r);
      V8<T> qf[8];
      float4 ln[4];
      read_q(r + 1, qf, ln);  // past the last block: a stale buffer, unused
      const int qs = qstart + r * 32;
      f32x16 p, sn = zero16();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(sc[i], cs, -sel(lc, i)));
        if (MASK && kj > qs + a.coff + crow(i, g)) p[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sn = Mfma<T>::mma(qf[ks], kv[ks], sn);
      float* X = &xp[r & 1][pr][0];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(X + k * 256 + lane * 4) =
            make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
      const V8<T> pf0 = cvt8s<T>(p, 0), pf1 = cvt8s<T>(p, 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = Mfma<T>::mma(dt[0][db], pf0, acc[db]);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = Mfma<T>::mma(dt[1][db], pf1, acc[db]);
      read_dt(r + 1, dt);  // past the last block: a stale buffer, unused
      sc = sn;
#pragma unroll
      for (int i = 0; i < 4; ++i) lc[i] = ln[i];
      tile_publish(r);
      __syncthreads();
    };
    int r = 0;
    for (; r < nmask; ++r) round(BoolTag<true>{}, r);
    for (; r < nblk; ++r) round(BoolTag<false>{}, r);
    if (nblk > 0) {  // round nblk: the partner's last dK block
      tile_issue(nblk);
      tile_publish(nblk);
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no buffer load outlives the workgroup
    if (kj < a.Sk) {
      T* dvrow = (T*)a.dv.p + b * a.dv.sb + h * a.dv.sh + (int64_t)kj * a.dv.ss;
      store_rows4(dvrow, acc, 1.f, g);
    }
  } else {
    // dO rows and -delta of block j (operands of dP(j) - delta).
    auto read_do = [&](int j, V8<T>* of, f32x16& d) {
      const T* D = qtile(j) + kTR;
      const int ro = rowoff(j);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) of[ks] = frag_r_swz(D, ro, ks * 2);
      const float* N = stats(j, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(N + i * 8 + g * 4);
        d[i * 4 + 0] = v.x; d[i * 4 + 1] = v.y; d[i * 4 + 2] = v.z; d[i * 4 + 3] = v.w;
      }
    };
    // Q^T of block j (operand of dK(j)).
    auto read_qt = [&](int j, V8<T> (*qt)[4]) {
      const T* Q = qtile(j);
      const int ro = rowoff(j);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db) qt[tt][db] = frag_t_swz(Q, ro, tt, db * 32);
    };
    f32x16 dc, dn;   // dP - delta of the previous block, and of this round's block
    V8<T> of[8];     // dO rows of this round's block (read before the barrier)
    V8<T> qt[2][4];  // Q^T of the previous block (read before the barrier)
    // Round r: dP(r) - delta (MFMA) while dS(r-1) = P(r-1) (dP(r-1) - delta)
    // is formed (VALU), then dK(r-1).  The next round's tile operands (dO
    // rows and -delta of block r+1, Q^T of block r) are read before the
    // barrier; only P waits for it.
    if (nblk > 0) {
      read_do(0, of, dn);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dn = Mfma<T>::mma(of[ks], kv[ks], dn);
      dc = dn;
      read_qt(0, qt);
      read_do(1, of, dn);  // past the last block: a stale buffer, unused
      tile_publish(0);
      __syncthreads();
    }
    for (int r = 1; r <= nblk; ++r) {
      tile_issue(r);
      const int j = r - 1;
      const float* X = &xp[j & 1][pr][0];
      f32x16 p;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = *reinterpret_cast<const float4*>(X + k * 256 + lane * 4);
        p[4 * k] = v.x; p[4 * k + 1] = v.y; p[4 * k + 2] = v.z; p[4 * k + 3] = v.w;
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dn = Mfma<T>::mma(of[ks], kv[ks], dn);
      f32x16 x;
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = p[i] * dc[i];
      const V8<T> sf0 = cvt8s<T>(x, 0), sf1 = cvt8s<T>(x, 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = Mfma<T>::mma(qt[0][db], sf0, acc[db]);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = Mfma<T>::mma(qt[1][db], sf1, acc[db]);
      dc = dn;
      read_qt(r, qt);          // past the last block: a stale buffer, unused
      read_do(r + 1, of, dn);  // likewise
      tile_publish(r);
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (kj < a.Sk) {
      T* dkrow = (T*)a.dk.p + b * a.dk.sb + h * a.dk.sh + (int64_t)kj * a.dk.ss;
      store_rows4(dkrow, acc, a.scale, g);
    }
  }
}

template <class T, bool CAUSAL>
hipError_t launch_split(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (((int64_t)a.Sk + kBN - 1) / kBN) * a.B * a.H;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dkdv_split_d128<T, CAUSAL>),
                         dim3((unsigned)grid), dim3(512), args, 0, s);
}

}  // namespace

// Byte offsets of every Q and dO row the split kernel may address (its last
// tile ends below Sq + 64) fit in 31 bits, and rows do not overlap.
bool dkdv_split_fits(const BwdArgs& a, int esize) {
  const int64_t lim = (int64_t)1 << 31;
  return a.q.ss >= kD && a.dout.ss >= kD && ((int64_t)a.Sq + kBM) * a.q.ss * esize < lim &&
         ((int64_t)a.Sq + kBM) * a.dout.ss * esize < lim;
}

int dkdv_split_lds() {
  return kNB * 2 * kTR * 2 + 2 * kNP * kXP * 4 + kNB * 2 * kBM * 4;
}

hipError_t launch_dkdv_split(const BwdArgs& a, int dtype, int causal, hipStream_t s) {
  if (dtype == 2)
    return causal ? launch_split<bf16_t, true>(a, s) : launch_split<bf16_t, false>(a, s);
  return causal ? launch_split<half_t, true>(a, s) : launch_split<half_t, false>(a, s);
}

}  // namespace fa
