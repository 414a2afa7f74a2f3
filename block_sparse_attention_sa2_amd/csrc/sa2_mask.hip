// Hybrid Top-k + Top-p block-mask builder (SpargeAttention2; gist.science,
// section 2A, with Top-p as the smallest set reaching cumulative mass p,
// section 1).
//
// Kernels on the caller's stream:
//   pool       q-bar / k-bar: fp64 means of each block's tokens (HBM stream)
//   score      S-bar = q-bar k-bar^T / sqrt(d), fp64, 64x64 tiles
//   select     one workgroup per query-block row: softmax, rank, cut, emit
//              the bitmap row, row count and ascending row list
//   columns    transposed lists (query blocks per key block), ascending
//   order      optional work orders (longest lists first)
// fp64 throughout keeps the ranking and the Top-p cut equal to an exact
// evaluation except where two scores, or the mass and p, agree to ~1e-15.
#include <math.h>

#include "sa2_common.h"

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
// score: S-bar tile of 64 query blocks x 64 key blocks per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void score_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar, int Tq,
                  int Tk, int d, double sqrt_d, double* __restrict__ sbar) {
  constexpr int TK = 32;  // d chunk
  __shared__ double qs[64][TK + 1];
  __shared__ double ks[64][TK + 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const double* qb = qbar + (size_t)bh * Tq * d;
  const double* kb = kbar + (size_t)bh * Tk * d;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
  for (int c0 = 0; c0 < d; c0 += TK) {
    for (int e = tid; e < 64 * TK; e += 256) {
      const int r = e / TK, c = e % TK;
      const int ii = i0 + r, jj = j0 + r, cc = c0 + c;
      qs[r][c] = (ii < Tq && cc < d) ? qb[(size_t)ii * d + cc] : 0.0;
      ks[r][c] = (jj < Tk && cc < d) ? kb[(size_t)jj * d + cc] : 0.0;
    }
    __syncthreads();
    const int kk_end = min(TK, d - c0);
    for (int kk = 0; kk < kk_end; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = qs[ty + 16 * a][kk];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = ks[tx + 16 * c][kk];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fma(av[a], bv[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int ii = i0 + ty + 16 * a;
    if (ii >= Tq) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int jj = j0 + tx + 16 * c;
      if (jj < Tk) sbar[((size_t)bh * Tq + ii) * Tk + jj] = acc[a][c] / sqrt_d;
    }
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

// Deterministic workgroup reductions (fixed combination order).
__device__ inline double wg_max(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < kMaskThreads / 64; ++i) r = fmax(r, red[i]);
  return r;
}
__device__ inline double wg_sum(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < kMaskThreads / 64; ++i) r += red[i];
  return r;
}
// Exclusive prefix over threads in thread order (values are small counts or
// fp64 masses); returns this thread's exclusive prefix, total in *total.
template <typename V>
__device__ inline V wg_exclusive_scan(V v, V* buf, V* total) {
  __syncthreads();
  buf[threadIdx.x] = v;
  __syncthreads();
  // Hillis-Steele over kMaskThreads entries, in LDS
  for (int off = 1; off < kMaskThreads; off <<= 1) {
    V add = (threadIdx.x >= off) ? buf[threadIdx.x - off] : V(0);
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  *total = buf[kMaskThreads - 1];
  return buf[threadIdx.x] - v;
}

// "a is ranked before b": higher score, lower index on ties.
__device__ inline bool ranks_before(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// One workgroup per (b*h, query block) row.  Dynamic LDS: P2 keys (u64),
// P2 indices (u32), Tk flags (u8), P2 = next power of two >= Tk.
__global__ __launch_bounds__(kMaskThreads)
void select_kernel(const double* __restrict__ sbar, int Tk, int P2, int kc, double p, int all,
                   uint8_t* __restrict__ bitmap, int32_t* __restrict__ row_cnt,
                   int32_t* __restrict__ row_idx) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);
  uint32_t* idx = reinterpret_cast<uint32_t*>(key + P2);
  uint8_t* flag = reinterpret_cast<uint8_t*>(idx + P2);
  __shared__ double red[kMaskThreads / 64];
  __shared__ double fscan[kMaskThreads];
  __shared__ int iscan[kMaskThreads];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const double* s = sbar + (size_t)row * Tk;

  int c;
  if (all) {
    c = Tk;
    for (int j = tid; j < Tk; j += kMaskThreads) flag[j] = 1;
  } else {
    // softmax statistics of the row
    double mx = -INFINITY;
    for (int j = tid; j < Tk; j += kMaskThreads) mx = fmax(mx, s[j]);
    mx = wg_max(mx, red);
    double z = 0.0;
    for (int j = tid; j < Tk; j += kMaskThreads) z += exp(s[j] - mx);
    z = wg_sum(z, red);
    // rank: bitonic sort of (key, index) pairs, padding last
    for (int j = tid; j < P2; j += kMaskThreads) {
      key[j] = (j < Tk) ? order_key(s[j]) : 0ull;
      idx[j] = (uint32_t)j;
    }
    for (int j = tid; j < Tk; j += kMaskThreads) flag[j] = 0;
    __syncthreads();
    for (int kk = 2; kk <= P2; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int t = tid; t < P2 / 2; t += kMaskThreads) {
          const int a = (t / jj) * 2 * jj + (t % jj);
          const int b = a + jj;
          const uint64_t ka = key[a], kb = key[b];
          const uint32_t ia = idx[a], ib = idx[b];
          const bool fwd = (a & kk) == 0;
          const bool a_first = ranks_before(ka, ia, kb, ib);
          if (fwd != a_first) {
            key[a] = kb; key[b] = ka;
            idx[a] = ib; idx[b] = ia;
          }
        }
        __syncthreads();
      }
    }
    // Top-p count: ranks r whose running mass (through r) is still below p
    int pc = 0;
    if (p >= 1.0) {
      pc = Tk;
    } else if (p > 0.0) {
      const int per = (P2 + kMaskThreads - 1) / kMaskThreads;
      const int r_lo = tid * per, r_hi = min(Tk, r_lo + per);
      double local = 0.0;
      for (int r = r_lo; r < r_hi; ++r) local += exp(key_value(key[r]) - mx) / z;
      double tot;
      double run = wg_exclusive_scan(local, fscan, &tot);
      int below = 0;
      for (int r = r_lo; r < r_hi; ++r) {
        run += exp(key_value(key[r]) - mx) / z;
        below += (run < p) ? 1 : 0;
      }
      int btot;
      (void)wg_exclusive_scan(below, iscan, &btot);
      pc = (btot < Tk) ? btot + 1 : Tk;
    }
    c = max(kc, pc);
    __syncthreads();
    for (int r = tid; r < c; r += kMaskThreads) flag[idx[r]] = 1;
  }
  __syncthreads();
  // emit the bitmap row and the ascending row list
  uint8_t* bm = bitmap + (size_t)row * Tk;
  for (int j = tid; j < Tk; j += kMaskThreads) bm[j] = flag[j];
  const int per = (Tk + kMaskThreads - 1) / kMaskThreads;
  const int j_lo = tid * per, j_hi = min(Tk, j_lo + per);
  int mine = 0;
  for (int j = j_lo; j < j_hi; ++j) mine += flag[j];
  int tot;
  int pos = wg_exclusive_scan(mine, iscan, &tot);
  int32_t* out = row_idx + (size_t)row * Tk;
  for (int j = j_lo; j < j_hi; ++j)
    if (flag[j]) out[pos++] = j;
  if (tid == 0) row_cnt[row] = c;
}

// ---------------------------------------------------------------------------
// columns: workgroup per (b*h, 64 key blocks); thread (part, column) counts
// its quarter of the query-block rows, then writes its entries at the prefix.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void columns_kernel(const uint8_t* __restrict__ bitmap, int Tq, int Tk,
                    int32_t* __restrict__ col_cnt, int32_t* __restrict__ col_idx) {
  __shared__ int cnt[4][64];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, c = tid % 64, part = tid / 64;
  const int j = blockIdx.x * 64 + c;
  const int per = (Tq + 3) / 4;
  const int i_lo = part * per, i_hi = min(Tq, i_lo + per);
  const uint8_t* bm = bitmap + (size_t)bh * Tq * Tk;
  int n = 0;
  if (j < Tk)
    for (int i = i_lo; i < i_hi; ++i) n += bm[(size_t)i * Tk + j];
  cnt[part][c] = n;
  __syncthreads();
  if (j >= Tk) return;
  int off = 0;
  for (int q = 0; q < part; ++q) off += cnt[q][c];
  int32_t* out = col_idx + ((size_t)bh * Tk + j) * Tq;
  for (int i = i_lo; i < i_hi; ++i)
    if (bm[(size_t)i * Tk + j]) out[off++] = i;
  if (part == 3) col_cnt[(size_t)bh * Tk + j] = off;
}

// ---------------------------------------------------------------------------
// Work orders.  Workgroup slot i of an attention kernel runs on XCD i % 8.
// XCD x takes the contiguous share of the natural (b, h, block) order that
// the fixed XCD-aware mapping (xcd_remap) gives it, so that its L2 sees the
// inputs of a narrow band of heads; within that share its slots are filled
// by decreasing list length, so that each XCD starts its longest lists first.
// One workgroup per (order, XCD) counts, scans and places in LDS; the order
// among equal counts is whatever the LDS atomics give (it affects scheduling
// only).
// ---------------------------------------------------------------------------
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads)
void order_kernel(const int32_t* __restrict__ row_cnt, int nrows, int row_max,
                  const int32_t* __restrict__ col_cnt, int ncols, int col_max,
                  int32_t* __restrict__ row_order, int32_t* __restrict__ col_order) {
  __shared__ int hist[kMaxTk + 1];
  __shared__ int scan[kOrderThreads];
  const int which = blockIdx.x / 8, x = blockIdx.x % 8;
  const int32_t* cnt = which == 0 ? row_cnt : col_cnt;
  int32_t* order = which == 0 ? row_order : col_order;
  const int n = which == 0 ? nrows : ncols;
  const int nb = (which == 0 ? row_max : col_max) + 1;   // counts 0 .. max
  // this XCD's share of the natural order (as in xcd_remap)
  const int qn = n / 8, rn = n % 8;
  const int c0 = x * qn + min(x, rn), len = qn + (x < rn ? 1 : 0);
  const int tid = threadIdx.x;
  for (int c = tid; c < nb; c += kOrderThreads) hist[c] = 0;
  __syncthreads();
  for (int j = tid; j < len; j += kOrderThreads) atomicAdd(&hist[cnt[c0 + j]], 1);
  __syncthreads();
  // first position of each count in descending-count order
  const int per = (nb + kOrderThreads - 1) / kOrderThreads;
  const int lo = tid * per, hi = min(nb, lo + per);   // positions in descending order
  int local = 0;
  for (int r = lo; r < hi; ++r) local += hist[nb - 1 - r];
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kOrderThreads; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int run = scan[tid] - local;
  for (int r = lo; r < hi; ++r) {
    const int c = nb - 1 - r;
    const int h = hist[c];
    hist[c] = run;
    run += h;
  }
  __syncthreads();
  // rank j within the share goes to slot 8j + x (slots i with i % 8 == x)
  for (int j = tid; j < len; j += kOrderThreads) {
    const int id = c0 + j;
    order[8 * atomicAdd(&hist[cnt[id]], 1) + x] = id;
  }
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

extern "C" sa2_status sa2_build_mask(const void* q, const void* k, int dtype, int B, int H, int N,
                                     int d, int bq, int bk, double k_frac, double p,
                                     const sa2_mask* m, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!q || !k || !m || !ws) return fail(SA2_EINVAL, "sa2_build_mask: null pointer");
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || bq <= 0 || bk <= 0)
    return fail(SA2_EINVAL, "sa2_build_mask: B, H, N, d, bq, bk must be positive");
  if (dtype != SA2_BF16 && dtype != SA2_F32)
    return fail(SA2_EINVAL, "sa2_build_mask: unknown dtype");
  if (d % 8 != 0 || d > 256)
    return fail(SA2_EUNSUPPORTED, "sa2_build_mask: d must be a multiple of 8 and at most 256");
  if (!aligned16(q) || !aligned16(k)) return fail(SA2_EINVAL, "sa2_build_mask: q/k not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(SA2_EINVAL, "sa2_build_mask: workspace not 256-byte aligned");
  if (std::isnan(k_frac) || std::isnan(p)) return fail(SA2_EINVAL, "sa2_build_mask: NaN k_frac or p");
  if (k_frac <= 0.0 && p <= 0.0)
    return fail(SA2_EINVAL, "sa2_build_mask: k_frac <= 0 and p <= 0 select nothing");
  const int Tq = cdiv(N, bq), Tk = cdiv(N, bk);
  if (m->B != B || m->H != H || m->N != N || m->bq != bq || m->bk != bk || m->Tq != Tq ||
      m->Tk != Tk)
    return fail(SA2_EINVAL, "sa2_build_mask: mask geometry does not match the call");
  if (!m->bitmap || !m->row_cnt || !m->row_idx || !m->col_cnt || !m->col_idx)
    return fail(SA2_EINVAL, "sa2_build_mask: mask array is null");
  if (Tk > kMaxTk) return fail(SA2_EUNSUPPORTED, "sa2_build_mask: more than 4096 key blocks");
  if (Tq > kMaxTk) return fail(SA2_EUNSUPPORTED, "sa2_build_mask: more than 4096 query blocks");
  const size_t need = sa2_mask_workspace_bytes(B, H, N, d, bq, bk);
  if (ws_bytes < need)
    return fail(SA2_EINVAL, "sa2_build_mask: workspace smaller than sa2_mask_workspace_bytes()");
  if ((size_t)B * H * Tq > 0x7fffffff || (size_t)B * H * (Tq + Tk) > 0x7fffffff)
    return fail(SA2_EUNSUPPORTED, "sa2_build_mask: too many blocks");

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
  const bool orders = m->row_order != nullptr && m->col_order != nullptr;

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

  score_kernel<<<dim3(cdiv(Tk, 64), cdiv(Tq, 64), BH), 256, 0, s>>>(qbar, kbar, Tq, Tk, d,
                                                                    sqrt((double)d), sbar);
  if (sa2_status st = check_launch("score_kernel")) return st;

  const int kc = topk_count(k_frac, Tk);
  const int all = (kc >= Tk || p >= 1.0) ? 1 : 0;
  const int P2 = next_pow2(Tk);
  const size_t lds = (size_t)P2 * (8 + 4) + ((Tk + 15) & ~15);
  select_kernel<<<BH * Tq, kMaskThreads, lds, s>>>(sbar, Tk, P2, kc, p, all, m->bitmap,
                                                   m->row_cnt, m->row_idx);
  if (sa2_status st = check_launch("select_kernel")) return st;

  columns_kernel<<<dim3(cdiv(Tk, 64), BH), 256, 0, s>>>(m->bitmap, Tq, Tk, m->col_cnt,
                                                        m->col_idx);
  if (sa2_status st = check_launch("columns_kernel")) return st;
  if (orders) {
    order_kernel<<<16, kOrderThreads, 0, s>>>(m->row_cnt, BH * Tq, Tk, m->col_cnt, BH * Tk, Tq,
                                             m->row_order, m->col_order);
    if (sa2_status st = check_launch("order_kernel")) return st;
  }
  return SA2_OK;
}
