// Hybrid Top-k + Top-p block-mask builder (SpargeAttention2; gist.science,
// section 2A, with Top-p as the smallest set reaching cumulative mass p,
// section 1).
//
// Kernels on the caller's stream:
//   pool       q-bar / k-bar: fp64 means of each block's tokens (HBM stream)
//   score      S-bar = q-bar k-bar^T / sqrt(d), fp64 MFMAs, 16x32 tiles per wave
//   select     one wave per query-block row: softmax, rank, cut, emit the
//              bitmap row, row count and ascending row list
//   columns    transposed lists (query blocks per key block), ascending
//   plan       the work plans of the attention kernels (sa2_plan.h)
// fp64 throughout keeps the ranking and the Top-p cut equal to an exact
// evaluation except where two scores, or the mass and p, agree to ~1e-15.
#include <math.h>

#include <mutex>
#include <string>

#include "sa2_common.h"
#include "sa2_plan.h"

namespace sa2 {

constexpr int kMaskThreads = 256;
constexpr int kMaxTk = 4096;

// ---------------------------------------------------------------------------
// pool: one workgroup per (b*h, block) of Q (first BH*Tq groups) or K.
// d/8 lanes cover a token's d elements with 16-byte loads; the token rows of
// the block are strided over the remaining thread index.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kMaskThreads)
void pool_kernel(const T* __restrict__ q, const T* __restrict__ k, int BH, int N, int d,
                 int bq, int bk, int Tq, int Tk, double* __restrict__ qbar,
                 double* __restrict__ kbar) {
  __shared__ double part[kMaskThreads * 8];
  const int nq = BH * Tq;
  int blk = blockIdx.x;
  const T* X;
  double* out;
  int b, T_;
  if (blk < nq) {
    X = q; out = qbar; b = bq; T_ = Tq;
  } else {
    blk -= nq; X = k; out = kbar; b = bk; T_ = Tk;
  }
  const int bh = blk / T_, i = blk % T_;
  const int lo = i * b;
  const int cnt = min(N, lo + b) - lo;
  const int lpr = d / 8;                    // lanes per token row
  const int rpi = kMaskThreads / lpr;       // token rows per iteration
  const int tid = threadIdx.x;
  const int c8 = tid % lpr, r0 = tid / lpr;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r0 < rpi) {
    const T* base = X + ((size_t)bh * N + lo) * d + c8 * 8;
#pragma unroll 4
    for (int r = r0; r < cnt; r += rpi) {
      double v[8];
      load8_f64(base + (size_t)r * d, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    // partial sums of token-row group r0, laid out [r0][d]
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0 * d + c8 * 8 + e] = acc[e];
  }
  __syncthreads();
  const int groups = min(rpi, cnt);
  for (int c = tid; c < d; c += kMaskThreads) {
    double s = 0.0;
    for (int g = 0; g < groups; ++g) s += part[g * d + c];
    out[((size_t)bh * T_ + i) * d + c] = s / (double)cnt;
  }
}

// ---------------------------------------------------------------------------
// score: S-bar = q-bar k-bar^T / sqrt(d) on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64).  Lane layout (measured): A[i][k] comes from lane
// i + 16k, B[k][j] from lane j + 16k, and D[i][j] lands in element i / 4 of
// lane j + 16 (i % 4).  One workgroup of four waves per 64 x 64 tile of
// S-bar, each wave a 32 x 32 sub-tile (four independent 16 x 16
// accumulators); q-bar and k-bar rows go through two LDS buffers, d in
// chunks of 32, the next chunk's loads in flight while a chunk's products
// run, rows padded by 16 bytes so that the 16 rows a read instruction touches
// fall in distinct banks.  For MFMA pair (2u, 2u + 1) lane l holds d indices
// 8u + 2(l / 16) and the next one, so each product is a fp64 sum over d in a
// fixed order.  A one-wave 16 x 32 version reading its operands from L2 was
// 12% slower at the 14B-shaped layer (312 against 273 us), and one LDS
// buffer of 64-index chunks 5% slower again in the whole mask build.
// ---------------------------------------------------------------------------
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kScoreTile = 64, kScoreChunk = 32;
constexpr int kScoreRow = kScoreChunk + 2;   // doubles per LDS row (16 bytes of padding)
constexpr int kScoreStage = kScoreTile * kScoreChunk / 2 / 256;   // f64x2 per thread and tensor

__global__ __launch_bounds__(256)
void score_tile_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar, int Tq,
                       int Tk, int d, double sqrt_d, double* __restrict__ sbar) {
  __shared__ __attribute__((aligned(16))) double qs[2][kScoreTile * kScoreRow];
  __shared__ __attribute__((aligned(16))) double ks[2][kScoreTile * kScoreRow];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.y;
  const int tk = (Tk + kScoreTile - 1) / kScoreTile;
  const int i0 = (blockIdx.x / tk) * kScoreTile, j0 = (blockIdx.x % tk) * kScoreTile;
  const int wi = (wv >> 1) * 32, wj = (wv & 1) * 32;   // this wave's sub-tile
  const int r = lane & 15, g = lane >> 4;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  const double* qh = qbar + (size_t)bh * Tq * d;
  const double* kh = kbar + (size_t)bh * Tk * d;
  // a chunk of 32 d indices (the last one possibly 8, 16 or 24) of rows i0..
  // and j0.. (past the end: the last row), 16 bytes per thread and step
  f64x2 rq[kScoreStage], rk[kScoreStage];
  auto load = [&](int c0) {
    const int dc = min(kScoreChunk, d - c0), per_row = dc / 2;
#pragma unroll
    for (int t = 0; t < kScoreStage; ++t) {
      const int x = tid + 256 * t;
      if (x < kScoreTile * per_row) {
        const int row = x / per_row, c = (x % per_row) * 2;
        rq[t] = *reinterpret_cast<const f64x2*>(qh + (size_t)min(i0 + row, Tq - 1) * d + c0 + c);
        rk[t] = *reinterpret_cast<const f64x2*>(kh + (size_t)min(j0 + row, Tk - 1) * d + c0 + c);
      }
    }
  };
  auto store = [&](int c0, int buf) {
    const int dc = min(kScoreChunk, d - c0), per_row = dc / 2;
#pragma unroll
    for (int t = 0; t < kScoreStage; ++t) {
      const int x = tid + 256 * t;
      if (x < kScoreTile * per_row) {
        const int row = x / per_row, c = (x % per_row) * 2;
        *reinterpret_cast<f64x2*>(&qs[buf][row * kScoreRow + c]) = rq[t];
        *reinterpret_cast<f64x2*>(&ks[buf][row * kScoreRow + c]) = rk[t];
      }
    }
  };
  load(0);
  store(0, 0);
  __syncthreads();
  int buf = 0;
  for (int c0 = 0; c0 < d; c0 += kScoreChunk) {
    const bool more = c0 + kScoreChunk < d;
    if (more) load(c0 + kScoreChunk);   // in flight while this chunk's products run
    const int dc = min(kScoreChunk, d - c0);
    const double* qb = qs[buf];
    const double* kb = ks[buf];
    for (int u = 0; u < dc / 8; ++u) {
      f64x2 av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        av[a] = *reinterpret_cast<const f64x2*>(qb + (wi + 16 * a + r) * kScoreRow + 8 * u + 2 * g);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = *reinterpret_cast<const f64x2*>(kb + (wj + 16 * b + r) * kScoreRow + 8 * u + 2 * g);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a][h], bv[b][h], acc[a][b], 0, 0, 0);
    }
    if (more) store(c0 + kScoreChunk, buf ^ 1);   // the other buffer: read a chunk ago, before the barrier
    __syncthreads();
    buf ^= 1;
  }
  // element e of lane l: row 4e + l / 16, column l % 16 of its 16 x 16 block
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + wi + 16 * a + 4 * e + g, j = j0 + wj + 16 * b + r;
        if (i < Tq && j < Tk) sbar[((size_t)bh * Tq + i) * Tk + j] = acc[a][b][e] / sqrt_d;
      }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------

// Order-preserving map of a double onto uint64 (larger value, larger key).
// -0.0 is folded onto +0.0 first so that equal values get equal keys.
__device__ inline uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ inline double key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

// "a is ranked before b": higher score, lower index on ties.
__device__ inline bool ranks_before(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// ---------------------------------------------------------------------------
// select, one wave per (b*h, query block) row.  The row's P2 = 64E ranking
// entries (P2 = max(64, next power of two >= Tk)) live in registers: entry
// i = E*lane + e in register e of lane i / E.  The bitonic network's strides
// below E exchange registers within a lane; larger strides exchange lanes at
// xor distance 1 .. 32 without going through LDS memory (see xor_lane), so
// the sort needs no LDS array and no barrier.  The wave's row flags live in
// LDS (private to the wave).
// ---------------------------------------------------------------------------
constexpr int kSelectWaves = 4;

// The value of lane (lane ^ d), d in {1, 2, 4, 8, 16, 32}: DPP quad
// permutations for 1 and 2, a swizzle (xor mask 4 within 32 lanes) for 4, a
// rotation of each 16-lane row by 8 for 8, and the row and half-wave swaps
// for 16 and 32 (each swap returns both partners; the lane picks the other's).
template <int D>
__device__ inline uint32_t xor_lane(uint32_t v, int lane) {
  if constexpr (D == 1) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);
  if constexpr (D == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);
  if constexpr (D == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101f);
  if constexpr (D == 8) return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false);
  if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  }
  if constexpr (D == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// One network stage whose partners are D lanes apart: every register of a
// lane meets the same register of its partner lane.
template <int E, int D>
__device__ inline void cross_lane_stage(uint64_t* key, uint32_t* idx, int lane, int kk) {
  const bool lower = (lane & D) == 0;
  const bool fwd = ((lane * E) & kk) == 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t plo = xor_lane<D>((uint32_t)key[e], lane);
    const uint32_t phi = xor_lane<D>((uint32_t)(key[e] >> 32), lane);
    const uint32_t pi = xor_lane<D>(idx[e], lane);
    const uint64_t pk = ((uint64_t)phi << 32) | plo;
    const bool mine_first = ranks_before(key[e], idx[e], pk, pi);
    if (lower != (fwd == mine_first)) {
      key[e] = pk;
      idx[e] = pi;
    }
  }
}

// One compare-exchange of entries at network positions a < b = a + stride:
// position a ends with the entry ranked first if `fwd`, else the other.
__device__ inline void cx(uint64_t& ka, uint32_t& ia, uint64_t& kb, uint32_t& ib, bool fwd) {
  if (fwd != ranks_before(ka, ia, kb, ib)) {
    const uint64_t tk = ka; ka = kb; kb = tk;
    const uint32_t ti = ia; ia = ib; ib = ti;
  }
}

template <int E, int J>
__device__ inline void in_lane_stage(uint64_t* key, uint32_t* idx, int lane, int kk) {
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((e & J) == 0) cx(key[e], idx[e], key[e + J], idx[e + J], ((lane * E + e) & kk) == 0);
}

// One network stage (block size KK, partner distance JJ entries), its
// lane distance and direction known at compile time.
template <int E, int KK, int JJ>
__device__ inline void net_stage(uint64_t* key, uint32_t* idx, int lane) {
  if constexpr (JJ >= E) {
    cross_lane_stage<E, JJ / E>(key, idx, lane, KK);
  } else {
    in_lane_stage<E, JJ>(key, idx, lane, KK);
  }
}
// The merge of blocks of KK entries (distances KK/2 .. 1), then the next
// block size up to KMAX, all unrolled.  Networks of more than 8 entries per
// lane are fenced stage by stage: scheduled across stages they held more
// registers (the 32-entry lane sort of the long-row kernel: 387 against 182
// VGPRs) and ran slower than the loop they replace.
template <int E, int KK, int JJ, int KMAX>
__device__ inline void net_from(uint64_t* key, uint32_t* idx, int lane) {
  net_stage<E, KK, JJ>(key, idx, lane);
  if constexpr (E > 8) __builtin_amdgcn_sched_barrier(0);   // stage by stage, as a loop would
  if constexpr (JJ > 1) {
    net_from<E, KK, JJ / 2, KMAX>(key, idx, lane);
  } else if constexpr (KK < KMAX) {
    net_from<E, 2 * KK, KK, KMAX>(key, idx, lane);
  }
}

// Bitonic network over a wave's 64E entries (entry E*lane + e in register e)
// into ranking order; unrolled up to 8 entries per lane, a loop over the
// stages beyond (where unrolling costs occupancy).
template <int E>
__device__ inline void sort_wave(uint64_t* key, uint32_t* idx, int lane) {
  if constexpr (E <= 8) {
    net_from<E, 2, 1, 64 * E>(key, idx, lane);
    return;
  }
  for (int kk = 2; kk <= 64 * E; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj >= E) {
        switch (jj / E) {   // lane distance
          case 1: cross_lane_stage<E, 1>(key, idx, lane, kk); break;
          case 2: cross_lane_stage<E, 2>(key, idx, lane, kk); break;
          case 4: cross_lane_stage<E, 4>(key, idx, lane, kk); break;
          case 8: cross_lane_stage<E, 8>(key, idx, lane, kk); break;
          case 16: cross_lane_stage<E, 16>(key, idx, lane, kk); break;
          default: cross_lane_stage<E, 32>(key, idx, lane, kk); break;
        }
      } else {
        if constexpr (E >= 2) if (jj == 1) in_lane_stage<E, 1>(key, idx, lane, kk);
        if constexpr (E >= 4) if (jj == 2) in_lane_stage<E, 2>(key, idx, lane, kk);
        if constexpr (E >= 8) if (jj == 4) in_lane_stage<E, 4>(key, idx, lane, kk);
        if constexpr (E >= 16) if (jj == 8) in_lane_stage<E, 8>(key, idx, lane, kk);
        if constexpr (E >= 32) if (jj == 16) in_lane_stage<E, 16>(key, idx, lane, kk);
        if constexpr (E >= 64) if (jj == 32) in_lane_stage<E, 32>(key, idx, lane, kk);
      }
    }
  }
}

// A lane's E entries among themselves into ranking order (unrolled up to 32
// entries, a loop over the stages beyond).
template <int E>
__device__ inline void sort_lane(uint64_t* key, uint32_t* idx) {
  if constexpr (E <= 32) {
    if constexpr (E >= 2) net_from<E, 2, 1, E>(key, idx, 0);
    return;
  }
  for (int kk = 2; kk <= E; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if constexpr (E >= 2) if (jj == 1) in_lane_stage<E, 1>(key, idx, 0, kk);
      if constexpr (E >= 4) if (jj == 2) in_lane_stage<E, 2>(key, idx, 0, kk);
      if constexpr (E >= 8) if (jj == 4) in_lane_stage<E, 4>(key, idx, 0, kk);
      if constexpr (E >= 16) if (jj == 8) in_lane_stage<E, 8>(key, idx, 0, kk);
      if constexpr (E >= 32) if (jj == 16) in_lane_stage<E, 16>(key, idx, 0, kk);
      if constexpr (E >= 64) if (jj == 32) in_lane_stage<E, 32>(key, idx, 0, kk);
    }
  }
}

// Lane 0's entry of a wave-uniform 64-bit value's first register.
__device__ inline uint64_t first_lane_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}

// Top-p count over entries in ranking order (rank E*lane + e), the first n
// of them real, given mass[e] = exp(S - mx) (0 for the others; divided by
// the row total z in place): the smallest prefix whose mass w / z, summed in ranking order in fp64,
// reaches p; -1 if the n entries do not reach it.
template <int E>
__device__ inline int topp_prefix(double* mass, int lane, int n, double z, double p) {
  double local = 0.0;   // the weights become masses in place
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mass[e] /= z;
    local += mass[e];
  }
  // exclusive scan of the lane totals over the wave
  double incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  double run = incl - local;
  int below = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    run += mass[e];
    below += (lane * E + e < n && run < p) ? 1 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) below += __shfl_xor(below, off);
  return below < n ? below + 1 : -1;
}

// topp_prefix with the masses recomputed from the sorted keys (mass
// exp(S - mx) / z), so that no array of them is held.
template <int E>
__device__ inline int topp_prefix_chunked(const uint64_t* key, int lane, int n, double mx,
                                          double z, double p) {
  auto mass = [&](int e) { return lane * E + e < n ? exp(key_value(key[e]) - mx) / z : 0.0; };
  double local = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) local += mass(e);
  double incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  double run = incl - local;
  int below = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    run += mass(e);
    below += (lane * E + e < n && run < p) ? 1 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) below += __shfl_xor(below, off);
  return below < n ? below + 1 : -1;
}

__device__ inline double wave_sum_f64(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Rows of up to 256 key blocks are sorted whole (E <= 4).  Longer rows keep
// only c = max(kc, pc) of their Tk blocks, so they first take candidates
// (CAND): the row's entries are spread over the lanes (entry j in lane j % 64,
// so neighbouring key blocks land in different lanes), each lane ranks its
// own E entries and offers its best C (4 for rows of up to 512 blocks, 8 for
// longer ones), and the 64 C candidates are sorted.  The candidates' first c
// are the row's first c exactly when every lane's best entry left out (its
// C+1-th) ranks after candidate c - 1.  Otherwise, or when c exceeds 64 C or
// the candidates' mass does not reach p, the whole row is sorted: in the same
// wave for rows of up to 512 blocks (their E entries are still in its
// registers), and for longer rows by a second launch of the whole-row sort
// (with `marked`) that finishes just the rows marked row_cnt = -1.  Either way
// the kept set is the one the full ranking gives.
//
// The selection of one row by wave threadIdx.x / 64 of a workgroup of NW
// waves: s points at the row's Tk scores (global or LDS memory); writes the
// bitmap row, the row count and the ascending row list of global row `row`.
// The wave's row flags live in LDS (private to the wave).
template <int E, bool CAND, int NW>
__device__ inline void select_row(const double* s, int row, int Tk, int kc, double p, int all,
                                  uint8_t* __restrict__ bitmap, int32_t* __restrict__ row_cnt,
                                  int32_t* __restrict__ row_idx) {
  constexpr int P2 = 64 * E;
  constexpr int C = E >= 16 ? 8 : E / 2;   // candidates per lane
  static_assert(!CAND || C < E, "a lane keeps some of its entries back");
  __shared__ uint8_t flags_all[NW][P2];
  const int lane = threadIdx.x & 63;
  uint8_t* flag = flags_all[threadIdx.x >> 6];

  for (int j = lane; j < P2; j += 64) flag[j] = all && j < Tk ? 1 : 0;
  wave_lds_sync();
  int c = Tk;
  if (!all) {
    uint64_t key[E];
    uint32_t idx[E];
    bool whole = true;   // sort the whole row
    if constexpr (CAND) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        key[e] = j < Tk ? order_key(s[j]) : 0ull;   // padding ranks last
        idx[e] = (uint32_t)j;
      }
      sort_lane<E>(key, idx);
      uint64_t ck[C];
      uint32_t ci[C];
#pragma unroll
      for (int e = 0; e < C; ++e) {
        ck[e] = key[e];
        ci[e] = idx[e];
      }
      sort_wave<C>(ck, ci, lane);
      const double mx = key_value(first_lane_u64(ck[0]));
      int pcc = 0;
      if (p > 0.0) {
        double z = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((int)idx[e] < Tk) z += exp(key_value(key[e]) - mx);
        z = wave_sum_f64(z);
        double w[C];
#pragma unroll
        for (int e = 0; e < C; ++e) w[e] = exp(key_value(ck[e]) - mx);
        pcc = topp_prefix<C>(w, lane, 64 * C, z, p);
      }
      const int cc = max(kc, pcc);
      if (pcc >= 0 && cc <= 64 * C) {
        // candidate cc - 1 against every lane's best entry left out
        const int r = cc - 1, src = r / C, er = r % C;
        uint64_t kv = ck[0];
        uint32_t iv = ci[0];
#pragma unroll
        for (int e = 1; e < C; ++e)
          if (e == er) {
            kv = ck[e];
            iv = ci[e];
          }
        const uint64_t kr =
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kv >> 32), src) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kv, src);
        const uint32_t ir = (uint32_t)__builtin_amdgcn_readlane((int)iv, src);
        if (!__any(ranks_before(key[C], idx[C], kr, ir))) {
          whole = false;
          c = cc;
#pragma unroll
          for (int e = 0; e < C; ++e)
            if (lane * C + e < c) flag[ci[e]] = 1;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = lane * E + e;
        key[e] = j < Tk ? order_key(s[j]) : 0ull;   // padding ranks last
        idx[e] = (uint32_t)j;
      }
    }
    if constexpr (CAND && E > 8) {
      if (whole) {   // left to the whole-row launch
        if (lane == 0) row_cnt[row] = -1;
        return;
      }
    }
    // rows of up to 512 blocks whose candidates fall short are sorted whole
    // here, from the same registers (a bitonic network takes any input order)
    if (!CAND || whole) {
      sort_wave<E>(key, idx, lane);
      int pc = 0;
      if (p >= 1.0) {
        pc = Tk;
      } else if (p > 0.0) {
        // the row maximum is rank 0's score
        const double mx = key_value(first_lane_u64(key[0]));
        int r;
        if constexpr (E <= 8) {   // each exponential once
          double w[E];
          double z = 0.0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            w[e] = lane * E + e < Tk ? exp(key_value(key[e]) - mx) : 0.0;
            z += w[e];
          }
          r = topp_prefix<E>(w, lane, Tk, wave_sum_f64(z), p);
        } else {   // long rows: in 8-entry chunks, taken twice (registers)
          double z = 0.0;
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (lane * E + e < Tk) z += exp(key_value(key[e]) - mx);
          z = wave_sum_f64(z);
          r = topp_prefix_chunked<E>(key, lane, Tk, mx, z, p);
        }
        pc = r < 0 ? Tk : r;
      }
      c = max(kc, pc);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane * E + e < c) flag[idx[e]] = 1;
    }
    wave_lds_sync();
  }
  // the bitmap row and the ascending row list from the flags
  uint8_t* bm = bitmap + (size_t)row * Tk;
  for (int j = lane; j < Tk; j += 64) bm[j] = flag[j];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) mine += flag[lane * E + e];
  int pos = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(pos, off);
    if (lane >= off) pos += up;
  }
  pos -= mine;
  int32_t* out = row_idx + (size_t)row * Tk;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (flag[lane * E + e]) out[pos++] = lane * E + e;
  if (lane == 0) row_cnt[row] = c;
}

template <int E, bool CAND>
__global__ __launch_bounds__(64 * kSelectWaves)
void select_wave_kernel(const double* __restrict__ sbar, int nrows, int Tk, int kc, double p,
                        int all, int marked, uint8_t* __restrict__ bitmap,
                        int32_t* __restrict__ row_cnt, int32_t* __restrict__ row_idx) {
  const int row = blockIdx.x * kSelectWaves + (threadIdx.x >> 6);
  if (row >= nrows) return;
  if (marked && row_cnt[row] != -1) return;   // settled by the candidate launch
  select_row<E, CAND, kSelectWaves>(sbar + (size_t)row * Tk, row, Tk, kc, p, all, bitmap,
                                    row_cnt, row_idx);
}

// ---------------------------------------------------------------------------
// columns: workgroup per (b*h, 16 key blocks); thread (part, column) counts
// its sixteenth of the query-block rows, then writes its entries at the
// prefix of the parts before it, so each list comes out ascending.  Up to
// 64 rows per part the bitmap is read once (a bit mask in a register).
// ---------------------------------------------------------------------------
constexpr int kColsPerGroup = 16, kColParts = 256 / kColsPerGroup;

__global__ __launch_bounds__(256)
void columns_kernel(const uint8_t* __restrict__ bitmap, int Tq, int Tk,
                    int32_t* __restrict__ col_cnt, int32_t* __restrict__ col_idx) {
  __shared__ int cnt[kColParts][kColsPerGroup];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, c = tid % kColsPerGroup, part = tid / kColsPerGroup;
  const int j = blockIdx.x * kColsPerGroup + c;
  const int per = (Tq + kColParts - 1) / kColParts;
  const int i_lo = part * per, i_hi = min(Tq, i_lo + per);
  const uint8_t* bm = bitmap + (size_t)bh * Tq * Tk;
  // up to 64 rows per part (Tq <= 1024): the part's flags are read once
  // into a bit mask, counted, and walked for the writes
  const bool in_regs = per <= 64;
  uint64_t flags = 0;
  int n = 0;
  if (j < Tk) {
    if (in_regs) {
      for (int i = i_lo; i < i_hi; ++i)
        flags |= (uint64_t)(bm[(size_t)i * Tk + j] != 0) << (i - i_lo);
      n = __popcll(flags);
    } else {
      for (int i = i_lo; i < i_hi; ++i) n += bm[(size_t)i * Tk + j];
    }
  }
  cnt[part][c] = n;
  __syncthreads();
  if (j >= Tk) return;
  int off = 0;
  for (int q = 0; q < part; ++q) off += cnt[q][c];
  int32_t* out = col_idx + ((size_t)bh * Tk + j) * Tq;
  if (in_regs) {
    while (flags) {
      out[off++] = i_lo + __ffsll((long long)flags) - 1;
      flags &= flags - 1;
    }
  } else {
    for (int i = i_lo; i < i_hi; ++i)
      if (bm[(size_t)i * Tk + j]) out[off++] = i;
  }
  if (part == kColParts - 1) col_cnt[(size_t)bh * Tk + j] = off;
}

// ---------------------------------------------------------------------------
// The mask's work plans (see sa2_plan.h), one workgroup per XCD share and
// kind of list: workgroups 0..7 the row plan, 8..15 the column plan (in a
// group planned head by head, the group's first workgroup plans all four).
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads)
void plan_kernel(const int32_t* __restrict__ row_cnt, int nrows, int Tk,
                 int32_t* __restrict__ row_plan, const int32_t* __restrict__ col_cnt, int ncols,
                 int Tq, int32_t* __restrict__ col_plan) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int itot[kPlanThreads / 64];
  __shared__ long long red[kPlanThreads / 64];
  __shared__ int ctr[6];
  __shared__ long long pos[20];
  const int x = blockIdx.x % 8;
  const bool rows = blockIdx.x < 8;
  const PlanKind kd = rows ? kRowPlan : kColPlan;
  const int n = rows ? nrows : ncols, ndone = rows ? kRowCounters : kColCounters;
  const PlanLayout l = plan_layout(n, kd, ndone);
  char* b = reinterpret_cast<char*>(rows ? row_plan : col_plan);
  plan_share(x, rows ? row_cnt : col_cnt, n, rows ? Tk : Tq, rows ? Tq : Tk, kd,
             reinterpret_cast<int4*>(b + l.items), reinterpret_cast<int4*>(b + l.splits),
             reinterpret_cast<int*>(b + l.done), ndone, hist, itot, red, ctr, pos);
}

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

static int topk_count(double k_frac, int Tk) {
  if (k_frac <= 0.0) return 0;
  if (k_frac >= 1.0) return Tk;
  const int c = (int)ceil(k_frac * (double)Tk - 1e-6);
  return min(Tk, max(1, c));
}

}  // namespace sa2

using namespace sa2;

extern "C" size_t sa2_mask_workspace_bytes(int B, int H, int N, int d, int bq, int bk) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || bq <= 0 || bk <= 0) return 0;
  const size_t BH = (size_t)B * H, Tq = cdiv(N, bq), Tk = cdiv(N, bk);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(BH * Tq * d * 8) + up(BH * Tk * d * 8) + up(BH * Tq * Tk * 8);
}

namespace sa2 {

// Arguments of a mask build that can be checked on the host alone (no
// workspace involved).
static sa2_status check_mask_args(const char* fn, const void* q, const void* k, int dtype, int B,
                                  int H, int N, int d, int bq, int bk, double k_frac, double p,
                                  const sa2_mask* m) {
  const std::string f(fn);
  if (!q || !k || !m) return fail(SA2_EINVAL, f + ": null pointer");
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || bq <= 0 || bk <= 0)
    return fail(SA2_EINVAL, f + ": B, H, N, d, bq, bk must be positive");
  if (dtype != SA2_BF16 && dtype != SA2_F32) return fail(SA2_EINVAL, f + ": unknown dtype");
  if (d % 8 != 0 || d > 256)
    return fail(SA2_EUNSUPPORTED, f + ": d must be a multiple of 8 and at most 256");
  if (!aligned16(q) || !aligned16(k)) return fail(SA2_EINVAL, f + ": q/k not 16-byte aligned");
  if (std::isnan(k_frac) || std::isnan(p)) return fail(SA2_EINVAL, f + ": NaN k_frac or p");
  if (k_frac <= 0.0 && p <= 0.0)
    return fail(SA2_EINVAL, f + ": k_frac <= 0 and p <= 0 select nothing");
  const int Tq = cdiv(N, bq), Tk = cdiv(N, bk);
  if (m->B != B || m->H != H || m->N != N || m->bq != bq || m->bk != bk || m->Tq != Tq ||
      m->Tk != Tk)
    return fail(SA2_EINVAL, f + ": mask geometry does not match the call");
  if (!m->bitmap || !m->row_cnt || !m->row_idx || !m->col_cnt || !m->col_idx || !m->row_plan ||
      !m->col_plan)
    return fail(SA2_EINVAL, f + ": mask array is null");
  if (!aligned16(m->row_plan) || !aligned16(m->col_plan))
    return fail(SA2_EINVAL, f + ": mask plans must be 16-byte aligned");
  if (Tk > kMaxTk) return fail(SA2_EUNSUPPORTED, f + ": more than 4096 key blocks");
  if (Tq > kMaxTk) return fail(SA2_EUNSUPPORTED, f + ": more than 4096 query blocks");
  if ((size_t)B * H * Tq > 0x7fffffff || (size_t)B * H * (Tq + Tk) > 0x7fffffff)
    return fail(SA2_EUNSUPPORTED, f + ": too many blocks");
  if ((size_t)B * H > 65535)   // (b, h) pairs index the second grid dimension
    return fail(SA2_EUNSUPPORTED, f + ": more than 65535 (batch, head) pairs");
  return SA2_OK;
}

// The launches of a mask build; arguments already checked, ws large enough.
static sa2_status launch_mask(const void* q, const void* k, int dtype, int B, int H, int N, int d,
                              int bq, int bk, double k_frac, double p, const sa2_mask* m,
                              void* ws, void* stream);

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is a file-scope device array.  Each
// GPU holds its own copy from module load until the process ends; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// device (kept per device below), never through the array's name.  Every
// call on one GPU uses the same array, so calls that overlap on one GPU
// (e.g. on two streams) race.  Nothing in it needs to start at zero: every
// byte a kernel reads was written earlier in the same call.
// ---------------------------------------------------------------------------
constexpr size_t kMaskScratchBytes = SA2_MASK_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kMaskScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The device address of `scratch` on `dev` (looked up once per device, with
// that device current).
static sa2_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA2_EUNSUPPORTED, "sa2_build_mask_noalloc: device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
      return fail(SA2_EDEVICE, "sa2_build_mask_noalloc: hipGetDevice failed");
    if (cur != dev && hipSetDevice(dev) != hipSuccess)
      return fail(SA2_EDEVICE, "sa2_build_mask_noalloc: hipSetDevice failed");
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(SA2_EDEVICE, std::string("sa2_build_mask_noalloc: hipGetSymbolAddress: ") +
                                   hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SA2_OK;
}

}  // namespace sa2

extern "C" sa2_status sa2_build_mask_noalloc(const void* q, const void* k, int dtype, int B,
                                             int H, int N, int d, int bq, int bk, double k_frac,
                                             double p, const sa2_mask* m, void* stream) {
  if (sa2_status st = check_mask_args("sa2_build_mask_noalloc", q, k, dtype, B, H, N, d, bq, bk,
                                      k_frac, p, m))
    return st;
  const size_t need = sa2_mask_workspace_bytes(B, H, N, d, bq, bk);
  if (need > kMaskScratchBytes)
    return fail(SA2_EUNSUPPORTED,
                "sa2_build_mask_noalloc: this geometry needs " + std::to_string(need) +
                    " bytes of workspace, more than the " + std::to_string(kMaskScratchBytes) +
                    " of the static scratch array; use sa2_build_mask with a workspace");
  int dev = -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(SA2_EDEVICE, "sa2_build_mask_noalloc: cannot tell the stream's device");
  void* ws = nullptr;
  if (sa2_status st = scratch_on(dev, &ws)) return st;
  return launch_mask(q, k, dtype, B, H, N, d, bq, bk, k_frac, p, m, ws, stream);
}

extern "C" size_t sa2_mask_plan_bytes(int B, int H, int N, int bq, int bk, int columns) {
  if (B <= 0 || H <= 0 || N <= 0 || bq <= 0 || bk <= 0 || (columns != 0 && columns != 1))
    return 0;
  const size_t n = (size_t)B * H * cdiv(N, columns ? bk : bq);
  if (n > 0x7fffffff) return 0;
  return columns ? plan_layout((int)n, kColPlan, kColCounters).bytes
                 : plan_layout((int)n, kRowPlan, kRowCounters).bytes;
}

extern "C" sa2_status sa2_mask_plans(const sa2_mask* m, void* stream) {
  if (!m) return fail(SA2_EINVAL, "sa2_mask_plans: null mask");
  if (m->B <= 0 || m->H <= 0 || m->N <= 0 || m->bq <= 0 || m->bk <= 0 ||
      m->Tq != cdiv(m->N, m->bq) || m->Tk != cdiv(m->N, m->bk))
    return fail(SA2_EINVAL, "sa2_mask_plans: inconsistent mask geometry");
  if ((size_t)m->B * m->H * (m->Tq + m->Tk) > 0x7fffffff)
    return fail(SA2_EUNSUPPORTED, "sa2_mask_plans: too many blocks");
  if (!m->row_cnt || !m->col_cnt || !m->row_plan || !m->col_plan)
    return fail(SA2_EINVAL, "sa2_mask_plans: mask array is null");
  if (!aligned16(m->row_plan) || !aligned16(m->col_plan))
    return fail(SA2_EINVAL, "sa2_mask_plans: mask plans must be 16-byte aligned");
  const int BH = m->B * m->H;
  plan_kernel<<<16, kPlanThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      m->row_cnt, BH * m->Tq, m->Tk, m->row_plan, m->col_cnt, BH * m->Tk, m->Tq, m->col_plan);
  return check_launch("plan_kernel");
}

extern "C" sa2_status sa2_build_mask(const void* q, const void* k, int dtype, int B, int H, int N,
                                     int d, int bq, int bk, double k_frac, double p,
                                     const sa2_mask* m, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (sa2_status st = check_mask_args("sa2_build_mask", q, k, dtype, B, H, N, d, bq, bk, k_frac,
                                      p, m))
    return st;
  if (!ws) return fail(SA2_EINVAL, "sa2_build_mask: null pointer");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(SA2_EINVAL, "sa2_build_mask: workspace not 256-byte aligned");
  if (ws_bytes < sa2_mask_workspace_bytes(B, H, N, d, bq, bk))
    return fail(SA2_EINVAL, "sa2_build_mask: workspace smaller than sa2_mask_workspace_bytes()");
  return launch_mask(q, k, dtype, B, H, N, d, bq, bk, k_frac, p, m, ws, stream);
}

namespace sa2 {
static sa2_status launch_mask(const void* q, const void* k, int dtype, int B, int H, int N, int d,
                              int bq, int bk, double k_frac, double p, const sa2_mask* m,
                              void* ws, void* stream) {
  const int Tq = cdiv(N, bq), Tk = cdiv(N, bk);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int BH = B * H;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* w = static_cast<char*>(ws);
  double* qbar = reinterpret_cast<double*>(w);
  w += up((size_t)BH * Tq * d * 8);
  double* kbar = reinterpret_cast<double*>(w);
  w += up((size_t)BH * Tk * d * 8);
  double* sbar = reinterpret_cast<double*>(w);
  w += up((size_t)BH * Tq * Tk * 8);

  const int nblk = BH * (Tq + Tk);
  if (dtype == SA2_BF16)
    pool_kernel<bf16_t><<<nblk, kMaskThreads, 0, s>>>(static_cast<const bf16_t*>(q),
                                                      static_cast<const bf16_t*>(k), BH, N, d, bq,
                                                      bk, Tq, Tk, qbar, kbar);
  else
    pool_kernel<float><<<nblk, kMaskThreads, 0, s>>>(static_cast<const float*>(q),
                                                     static_cast<const float*>(k), BH, N, d, bq, bk,
                                                     Tq, Tk, qbar, kbar);
  if (sa2_status st = check_launch("pool_kernel")) return st;

  score_tile_kernel<<<dim3(cdiv(Tq, kScoreTile) * cdiv(Tk, kScoreTile), BH), 256, 0, s>>>(
      qbar, kbar, Tq, Tk, d, sqrt((double)d), sbar);
  if (sa2_status st = check_launch("score_tile_kernel")) return st;

  const int kc = topk_count(k_frac, Tk);
  const int all = (kc >= Tk || p >= 1.0) ? 1 : 0;
  const int P2 = max(64, next_pow2(Tk));
  const int rows = BH * Tq, sgrid = cdiv(rows, kSelectWaves), sthreads = 64 * kSelectWaves;
#define SA2_SELECT(E_, CAND_, MARKED_)                                                        \
  select_wave_kernel<E_, CAND_><<<sgrid, sthreads, 0, s>>>(sbar, rows, Tk, kc, p, all, MARKED_,   \
                                                          m->bitmap, m->row_cnt, m->row_idx)
#define SA2_SELECT_LONG(E_)                                                                   \
  SA2_SELECT(E_, true, 0);                                                                     \
  SA2_SELECT(E_, false, 1)
  switch (P2 / 64) {
    case 1: SA2_SELECT(1, false, 0); break;
    case 2: SA2_SELECT(2, false, 0); break;
    case 4: SA2_SELECT(4, false, 0); break;
    case 8: SA2_SELECT(8, true, 0); break;
    case 16: SA2_SELECT_LONG(16); break;
    case 32: SA2_SELECT_LONG(32); break;
    default: SA2_SELECT_LONG(64); break;
  }
#undef SA2_SELECT_LONG
#undef SA2_SELECT
  if (sa2_status st = check_launch("select_wave_kernel")) return st;

  columns_kernel<<<dim3(cdiv(Tk, kColsPerGroup), BH), 256, 0, s>>>(m->bitmap, Tq, Tk,
                                                                    m->col_cnt, m->col_idx);
  if (sa2_status st = check_launch("columns_kernel")) return st;
  plan_kernel<<<16, kPlanThreads, 0, s>>>(m->row_cnt, BH * Tq, Tk, m->row_plan, m->col_cnt,
                                          BH * Tk, Tq, m->col_plan);
  return check_launch("plan_kernel");
}
}  // namespace sa2
