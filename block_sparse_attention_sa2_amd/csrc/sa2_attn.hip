// Block-sparse attention, forward and backward (SpargeAttention2:
// gist.science section 2C — whole tiles are kept or dropped and dropped tiles
// cost neither matmul nor softmax; abstract item ii — the sparse attention is
// trainable, so the backward runs over the same mask).
//
// Tiles: a query block of bq = 64 or 128 rows per workgroup (32 rows per
// wave), key tiles of 64 tokens staged through LDS, bf16 MFMA 32x32x16 with
// fp32 accumulation, online softmax in base 2 with the 1/sqrt(d) scale and
// log2(e) folded into one multiplier.
//
// Orientation: the forward and dQ kernels compute S^T = K Q^T, so each lane
// owns one query row (its softmax statistics stay in the lane, with one
// exchange across the two half-waves), and the outputs are produced
// transposed (O^T = V^T P^T, dQ^T = K^T dS^T).  The V^T and K^T operands are
// read straight from row-major LDS tiles with ds_read_b64_tr_b16.
//
// Backward: the dQ kernel first (one workgroup per query block over its row
// list; it also forms Delta = rowsum(dO * O) and the log2-scaled LSE of its
// rows and leaves them in the workspace), then the dK/dV kernel (key blocks
// walking the query blocks of their column lists).
//
// Kernels: fwd_async_kernel, dq_async_kernel and dkdv_pair_kernel serve bf16
// and d = 128 (K/V tiles and Q/dO slices copied straight to LDS through
// buffer resources, double-buffered); with 64-row query blocks the forward
// and dQ run fwd_async32_kernel and dq_async32_kernel, which stage 32-key
// tiles so that twice as many workgroups fit a CU.  They walk the mask's
// work plans (the row plan for the forward and dQ, the column plan for
// dK/dV; see sa2_plan.h): a list longer than a fair share is cut into
// segments whose partial results the list's last segment combines in
// order.  fwd_kernel, dq_kernel and dkdv_kernel, staged through registers,
// serve fp32 inputs and d = 64 (in dkdv_kernel each wave owns a 32-row slice
// of every listed query block and the four partial tiles are summed in LDS
// in a fixed order).  On these paths no value is accumulated atomically, so
// the results are bitwise reproducible; the fused variant of
// sa2_attn_bwd_atomic_dq is the one exception (dQ added with fp32 atomics).
#include <math.h>

#include "sa2_common.h"
#include "sa2_plan.h"

namespace sa2 {

// LDS layouts of a 64-row tile of bf16 rows of D elements, chosen by how the
// tile is read (a wave64 LDS access is served 16 lanes or 32 lanes at a time):
//   kRows  16-byte MFMA fragments, 16 lanes reading one 16-byte unit of 16
//          consecutive rows: rows padded by 8 elements (a stride of 4 mod 64
//          banks), so the 16 units land on distinct banks;
//   kCols  transposed reads, 32 lanes reading 4 consecutive rows x 64 bytes:
//          rows padded by 32 elements (a stride of 16 mod 64 banks);
//   kBoth  read both ways: for D = 128 unpadded rows, with unit u of row r
//          stored at unit u ^ (4(r % 4) + (r / 4) % 4), which is conflict-free
//          for both patterns; for other D, padded by 16 elements;
//   kPad16 read both ways, rows padded by 16 elements (2-way conflicts on
//          both patterns, but no address registers).
// Padded layouts keep every per-step address a compile-time offset from one
// per-lane base; the permuted one costs a few address registers, which the
// dQ kernel cannot spare.
enum Layout { kRows = 0, kCols = 1, kBoth = 2, kPad16 = 3 };

template <int D, int L>
struct Tile {
  static constexpr bool kSwizzled = L == kBoth && D == 128;
  static constexpr int kRowElems =
      L == kRows ? D + 8 : L == kCols ? D + 32 : kSwizzled ? D : D + 16;
  __device__ static inline int off(int r, int col) {
    if constexpr (kSwizzled) {
      const int sw = ((r & 3) << 2) | ((r >> 2) & 3);
      return r * D + (((col >> 3) ^ sw) << 3) + (col & 7);
    } else {
      return r * kRowElems + col;
    }
  }
};

// ---------------------------------------------------------------------------
// Tile staging: rows key0 .. key0+63 of a [N, D] head, zero past N.
// ---------------------------------------------------------------------------
template <typename T, int D, int NT>
__device__ inline void fetch_tile(const T* __restrict__ x, int key0, int N, int tid, bf16x8* r) {
  constexpr int CPR = D / 8, CPT = 64 * CPR / NT;
  static_assert(CPT * NT == 64 * CPR, "tile chunks must divide evenly");
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT, row = ch / CPR, c8 = ch % CPR;
    const int key = key0 + row;
    r[c] = (unsigned)key < (unsigned)N ? load8(x + (size_t)key * D + c8 * 8) : zero8();
  }
}

template <int D, int L, int NT>
__device__ inline void put_tile(uint16_t* lds, int tid, const bf16x8* r) {
  constexpr int CPR = D / 8, CPT = 64 * CPR / NT;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT, row = ch / CPR, c8 = ch % CPR;
    *reinterpret_cast<bf16x8*>(lds + Tile<D, L>::off(row, c8 * 8)) = r[c];
  }
}

// A operand X^T[n][k-slots] of a 32x32x16 MFMA from a row-major LDS tile X,
// for the 16 rows k = kbase .. kbase+15 and the 32 columns n = nbase ..
// nbase+31.  Slot 8h + i (h = lane/32) maps to row kbase + 8(i/4) + 4h + i%4,
// the same order in which a 32x32 accumulator holds its rows, so an
// accumulator tile can be fed as the B operand.
template <int D, int L>
__device__ inline bf16x8 tr_operand(const uint16_t* lds, int kbase, int nbase, int lane) {
  const int h = lane >> 5;
  const int r = kbase + 4 * h + ((lane & 15) >> 2);
  const int c = nbase + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const bf16x4 lo = lds_read_tr(lds + Tile<D, L>::off(r, c));
  const bf16x4 hi = lds_read_tr(lds + Tile<D, L>::off(r + 8, c));
  return cat(lo, hi);
}

// Rows of the running max only move when the tile maximum exceeds them by
// more than this (log2 units): P then stays below 2^8, and the rescale of the
// output accumulators is skipped on most tiles.
constexpr float kRescaleThreshold = 8.0f;

// Eight accumulator values e0 .. e0+7 as a bf16 B operand.
__device__ inline bf16x8 pack8(const f32x16& a, int e0) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)a[e0 + i];
  return r;
}

// ---------------------------------------------------------------------------
// Byte offsets into a permuted tile (kBoth layout, d = 128: rows of 256
// bytes, 16-byte unit u of row r stored at u ^ swz(r)), for the two access
// patterns of the MFMA operands, each formed with one xor per read.
//   Row reads (A operand rows r = 32blk + l32, units 2kk + h):
//     (2kk + h) ^ swz(l32) = 2kk ^ (h ^ swz(l32)) -> ra ^ 32kk, + 8192blk.
//   Transposed reads (tr_operand: rows 16t + 4h + a (+8 for the high half),
//   a = (lane % 16) / 4, units 4db + c, c = 2((lane / 16) % 2) + (lane % 4) / 2):
//     the unit is 4(db ^ a) + (c ^ b), b = (h + 2hi) % 4 -> tb[hi] ^ 64db,
//     + 4096t.
// A kernel re-makes the bases opaque once per step (fresh()), so that the
// compiler forms each address in the loop instead of keeping one register
// per distinct address for the whole kernel.
// ---------------------------------------------------------------------------
struct SwzAddr {
  uint32_t ra, tb[2];
  __device__ explicit SwzAddr(int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    ra = 256u * l32 + 16u * (h ^ (((l32 & 3) << 2) | ((l32 >> 2) & 3)));
    const int a = (lane & 15) >> 2;
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      tb[hi] = 256u * (4 * h + a + 8 * hi) + 64u * a + 16u * (c ^ ((h + 2 * hi) & 3)) +
               8u * (lane & 1);
  }
  __device__ SwzAddr fresh() const {
    SwzAddr r = *this;
    asm volatile("" : "+v"(r.ra), "+v"(r.tb[0]), "+v"(r.tb[1]));
    return r;
  }
  __device__ uint32_t row(int blk, int kk) const { return 8192u * blk + (ra ^ (32u * kk)); }
  __device__ uint32_t tr(int t, int db, int hi) const {
    return (tb[hi] ^ (64u * db)) + 4096u * t;
  }
};
__device__ inline bf16x8 rd_row(const uint16_t* tile, uint32_t boff) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + boff);
}
// tr_operand<128, kBoth>(tile, 16t, 32db, lane) through the bases above
__device__ inline bf16x8 rd_tr(const uint16_t* tile, const SwzAddr& A, int t, int db) {
  const char* b = reinterpret_cast<const char*>(tile);
  return cat(lds_read_tr(reinterpret_cast<const uint16_t*>(b + A.tr(t, db, 0))),
             lds_read_tr(reinterpret_cast<const uint16_t*>(b + A.tr(t, db, 1))));
}

// Eight terms of Delta_t = sum_c dO_tc O_tc: O as stored, dO as the bf16
// MFMA operand it enters dP = dO V^T with (for fp32 inputs the rounded
// values), so that dP - Delta cancels exactly where the row's P is one-hot.
template <typename T>
__device__ inline float delta_part(const T* o8, bf16x8 dof) {
  float a[8];
  load8_f32(o8, a);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] * (float)dof[i];
  return s;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1, 2)))
void fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ row_cnt, const int32_t* __restrict__ row_idx,
                int N, int Tq, int Tk, float scale_log2,
                T* __restrict__ o, float* __restrict__ lse) {
  constexpr int NT = NW * 64;
  using KT = Tile<D, kRows>;
  using VT = Tile<D, kCols>;
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int CPT = 64 * (D / 8) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[64 * KT::kRowElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[64 * VT::kRowElems];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const T* kh = k + base;
  const T* vh = v + base;
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  bf16x8 qf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    qf[kk] = qvalid ? load8(q + base + (size_t)qrow * D + 16 * kk + 8 * h) : zero8();

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();
  float m = -INFINITY, lsum = 0.f;

  const int cnt = list_len(row_cnt[wg], Tk);
  const int32_t* lst = row_idx + (size_t)wg * Tk;
  bf16x8 kr[CPT], vr[CPT];
  if (cnt > 0) {
    fetch_tile<T, D, NT>(kh, lst[0] * 64, N, tid, kr);
    fetch_tile<T, D, NT>(vh, lst[0] * 64, N, tid, vr);
  }
  for (int t = 0; t < cnt; ++t) {
    const int key0 = lst[t] * 64;
    __syncthreads();
    put_tile<D, kRows, NT>(k_lds, tid, kr);
    put_tile<D, kCols, NT>(v_lds, tid, vr);
    __syncthreads();
    if (t + 1 < cnt) {
      const int nk0 = lst[t + 1] * 64;
      fetch_tile<T, D, NT>(kh, nk0, N, tid, kr);
      fetch_tile<T, D, NT>(vh, nk0, N, tid, vr);
    }
    // S^T for keys key0 .. key0+63 (two 32-key halves) against this lane's query
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = zero16();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        s[b] = mfma32(lds_read8(k_lds + KT::off(32 * b + l32, 16 * kk + 8 * h)), qf[kk], s[b]);
    }
    if (key0 + 64 > N) {  // the partial last key block (a uniform branch)
      const int lim = N - key0 - 4 * h;   // keys of this lane at offsets >= lim are past N
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + 8 * (e >> 2) + (e & 3) >= lim) s[b][e] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[b][e]);
    mx = wave_max32(mx) * scale_log2;
    if (__any(mx > m + kRescaleThreshold)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) acc[db] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][e], scale_log2, -m));
        s[b][e] = pv;
        ps += pv;
      }
    lsum += ps;
    // O^T += V^T P^T over four 16-key steps.  For fp32 inputs P enters as a
    // pair of bf16 terms (its rounding and the rounding's residual), so that
    // O carries P to about 16 bits rather than bf16's 8.
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const bf16x8 pf = pack8(s[tt >> 1], 8 * (tt & 1));
#pragma unroll
      for (int db = 0; db < ND; ++db)
        acc[db] = mfma32(tr_operand<D, kCols>(v_lds, 16 * tt, 32 * db, lane), pf, acc[db]);
      if constexpr (sizeof(T) == 4) {
        bf16x8 lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = (__bf16)(s[tt >> 1][8 * (tt & 1) + i] - (float)pf[i]);
#pragma unroll
        for (int db = 0; db < ND; ++db)
          acc[db] = mfma32(tr_operand<D, kCols>(v_lds, 16 * tt, 32 * db, lane), lo, acc[db]);
      }
    }
  }
  const float ltot = wave_sum32(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qvalid) {
    T* orow = o + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(orow + 32 * db + 8 * g + 4 * h, acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
               acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
    if (h == 0)
      lse[(size_t)bh * N + qrow] = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Asynchronous tile copies (bf16, d = 128), global -> LDS through buffer
// resources.  Rows of 256 bytes are copied in groups of four: lane l's 16
// bytes of group i land in LDS unit 64i + l, i.e. row 4i + l/16 and unit
// l % 16, which in the permuted kBoth layout holds the logical unit
// (l % 16) ^ swz(row).  swz(4i + l/16) = 4(l/16) + i % 4, so the lane's
// source offset within its group depends only on i % 4: four per-lane
// constants (unit_offsets) and an immediate 1024 (i % 4) serve every copy.
// Rows past N read as zeros (the resource ends at row N).
// ---------------------------------------------------------------------------
__device__ inline void unit_offsets(int lane, uint32_t* uo) {
  const int rr = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) uo[j] = rr * 256 + 16 * ((lane & 15) ^ ((rr << 2) | j));
}

// Groups g0 .. g0+4G-1 of the rows starting at row0 of a head (256-byte
// rows), into dst (the tile's LDS base).  g0 and row0 are wave-uniform.
template <int G>
__device__ inline void copy_groups(rsrc_t r, int row0, int g0, uint16_t* dst,
                                   const uint32_t* uo) {
  static_for<0, G>([&](auto jj) {
    constexpr int J = decltype(jj)::value;
    const int g = g0 + 4 * J;
    const uint32_t soff = (uint32_t)(row0 + 4 * g) * 256u;
    uint16_t* d = dst + g * 512;
    static_for<0, 4>([&](auto ii) {
      constexpr int I = decltype(ii)::value;
      buf_lds16<1024 * I>(r, d, uo[I], soff);
    });
  });
}

// A 64-key tile of K and of V: each of the NW waves copies 16 / NW groups.
template <int NW>
__device__ inline void copy_kv_tile(rsrc_t rk, rsrc_t rv, int key0, uint16_t* kdst,
                                    uint16_t* vdst, int w, const uint32_t* uo) {
  constexpr int PER = 16 / NW;
  static_assert(PER % 4 == 0, "a wave copies whole runs of four groups");
  copy_groups<PER / 4>(rk, key0, w * PER, kdst, uo);
  copy_groups<PER / 4>(rv, key0, w * PER, vdst, uo);
}

// Step loops over LDS rings.  The buffers of a ring are separate LDS arrays
// and the loop is unrolled by a multiple of the ring sizes, so that each step
// names its buffers statically and every LDS address is a register plus an
// immediate offset.
template <int P, typename F>
__device__ inline void unrolled_steps(int cnt, F&& step) {
  for (int t = 0; t < cnt; t += P)
    static_for<0, P>([&](auto j) {
      if (t + decltype(j)::value < cnt) step(t + decltype(j)::value, j);
    });
}
// Double buffering: one workgroup barrier per step; after it, every wave's
// copy for this step has landed (each waits for its own first) and every
// wave is done with the other buffer, which then receives the next copy.
template <typename F>
__device__ inline void double_buffered(int cnt, F&& step) {
  unrolled_steps<2>(cnt, step);
}

// s_waitcnt with vmcnt(VM) and lgkmcnt(0) (expcnt not waited).
template <int VM>
__device__ inline void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// Forward for bf16 and d = 128 with double-buffered asynchronous K/V tiles
// (see double_buffered).  The LDS operands of each MFMA group are read well
// ahead of their MFMAs (sched_group_barrier fixes the issue order), so that
// LDS latency overlaps the matrix work instead of stalling it.
//
// One workgroup per item of the row plan: a query block's row list, or one
// segment of a long one.  A segment leaves its unnormalised fp32 O^T rows,
// running maximum m and row sum l in a partial slot; the last segment of the
// row combines the slots in segment order:
//   M = max_s m_s,  l = sum_s l_s 2^(m_s - M),  O = sum_s O_s 2^(m_s - M) / l,
//   LSE = (M + log2 l) ln 2,
// which is the softmax over the whole row (each segment's m and O_s, l_s are
// consistent under the lazy rescale, whatever m it settled on).
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1, 2)))
void fwd_async_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ v, const int32_t* __restrict__ row_idx,
                      const int4* __restrict__ items, const int4* __restrict__ splits,
                      int* __restrict__ done, float* __restrict__ partials, int nrows, int N,
                      int Tq, int Tk, float scale_log2, bf16_t* __restrict__ o,
                      float* __restrict__ lse) {
  constexpr int D = 128;
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int TILE = 64 * D;
  constexpr int KCOPIES = 16 / NW;   // copy instructions per wave per tile tensor
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) uint16_t kb0[TILE], kb1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[TILE], vb1[TILE];
  __shared__ int last_segment;

  const int4 item = items[blockIdx.x];
  int4 sp;
  if (!plan_item_ok(item, nrows, Tk, kRowPlan, splits, sp)) return;
  const int wg = item.x;
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const rsrc_t rk = make_rsrc(k + base, (uint32_t)N * D * 2);
  const rsrc_t rv = make_rsrc(v + base, (uint32_t)N * D * 2);
  uint32_t uo[4];
  unit_offsets(lane, uo);
  const SwzAddr addr0(lane);
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  // this wave's 32 query rows are copied whole into the second K/V buffers
  // (free until step 0 issues its copy) and read from there in the MFMA
  // operand layout; rows past N arrive as zeros
  uint16_t* qs = (w < 2 ? kb1 : vb1) + (w & 1) * 32 * D;
  copy_groups<2>(make_rsrc(q + base, (uint32_t)N * D * 2), qi * BQ + w * 32, 0, qs, uo);

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();
  float m = -INFINITY, lsum = 0.f;

  // the list (segment) is walked with scalar loads, one entry ahead of its copy
  const int cnt = item.z;
  const int32_t* lst = row_idx + (size_t)wg * Tk + item.y;
  auto key_at = [&](int t) { return t < cnt ? lst[t] * 64 : 0; };
  int key_cur = key_at(0);
  if (cnt > 0) copy_kv_tile<NW>(rk, rv, key_cur, kb0, vb0, w, uo);
  int key_nxt = key_at(1);
  // the Q copy went out before the first tile's 2 * 16 / NW copy instructions
  if (cnt > 0) wait_vm_lgkm0<2 * (16 / NW)>();
  else wait_vm_lgkm0<0>();
  wave_lds_sync();
  bf16x8 qf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) qf[kk] = rd_row(qs, addr0.row(0, kk));

  double_buffered(cnt, [&](int t, auto parity) {
    constexpr bool odd = decltype(parity)::value == 1;
    const uint16_t* kt = odd ? kb1 : kb0;
    const uint16_t* vt = odd ? vb1 : vb0;
    const int key0 = key_cur;
    wait_vm_lgkm0<0>();
    __syncthreads();
    if (t + 1 < cnt) copy_kv_tile<NW>(rk, rv, key_nxt, odd ? kb0 : kb1, odd ? vb0 : vb1, w, uo);
    key_cur = key_nxt;
    key_nxt = key_at(t + 2);
    const SwzAddr A = addr0.fresh();

    // S = K Q^T: the first half's eight K fragments are read first, the
    // second half's are read while the first half's MFMAs run
    f32x16 s[2] = {zero16(), zero16()};
    {
      bf16x8 ka[NK], kc[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) ka[kk] = rd_row(kt, A.row(0, kk));
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        s[0] = mfma32(ka[kk], qf[kk], s[0]);
        kc[kk] = rd_row(kt, A.row(1, kk));
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) s[1] = mfma32(kc[kk], qf[kk], s[1]);
      __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);   // DS reads
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NK, 0);
    }
    if (key0 + 64 > N) {  // the partial last key block (a uniform branch)
      const int lim = N - key0 - 4 * h;   // keys of this lane at offsets >= lim are past N
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + 8 * (e >> 2) + (e & 3) >= lim) s[b][e] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[b][e]);
    mx = wave_max32(mx) * scale_log2;
    if (__any(mx > m + kRescaleThreshold)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) acc[db] *= alpha;
    }
    // the first V fragments are read while P is formed
    bf16x8 va[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) va[db] = rd_tr(vt, A, 0, db);
    float ps = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][e], scale_log2, -m));
        pf[2 * b + (e >> 3)][e & 7] = (__bf16)pv;
        ps += pv;
      }
    lsum += ps;
    // O^T += V^T P^T, the next 16-key step's V fragments read during this one's
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      bf16x8 vn[ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        acc[db] = mfma32(va[db], pf[tt], acc[db]);
        if (tt < 3) vn[db] = rd_tr(vt, A, tt + 1, db);
      }
      if (tt < 3)
#pragma unroll
        for (int db = 0; db < ND; ++db) va[db] = vn[db];
    }
  });

  const float ltot = wave_sum32(lsum);
  if (item.w < 0) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    bf16_t* orow = o + base + (size_t)(qvalid ? qrow : 0) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) store_row32(orow + 32 * db, acc[db], inv, h, qvalid);
    if (qvalid && h == 0)
      lse[(size_t)bh * N + qrow] = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
    return;
  }
  // one segment of a split row: O^T rows, m and l into its partial slot
  // ([BQ rows][D] unnormalised O, then m[BQ], l[BQ])
  const int entry = item.w >> 10, seg = item.w & 1023;
  {
    const int r = w * 32 + l32;
    float* part = partials + (size_t)(sp.y + seg) * kFwdPartialFloats;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(part + (size_t)r * D + 32 * db + 8 * g + 4 * h, acc[db][4 * g],
               acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]);
    part[(size_t)BQ * D + (h == 0 ? r : BQ + r)] = h == 0 ? m : ltot;
  }
  // release the partial, count this segment done; the last one combines
  __threadfence();
  __syncthreads();
  if (tid == 0) last_segment = atomicAdd(&done[entry], 1) == sp.z - 1;
  __syncthreads();
  if (!last_segment) return;
  __threadfence();
  // two threads per row, each half of its D columns
  const int r = tid >> 1, c0 = (tid & 1) * (D / 2);
  const float* part0 = partials + (size_t)sp.y * kFwdPartialFloats;
  float M = -INFINITY;
  for (int s2 = 0; s2 < sp.z; ++s2)
    M = fmaxf(M, part0[(size_t)s2 * kFwdPartialFloats + (size_t)BQ * D + r]);
  float osum[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) osum[c] = 0.f;
  float lt = 0.f;
  if (M > -INFINITY) {
    for (int s2 = 0; s2 < sp.z; ++s2) {
      const float* ps = part0 + (size_t)s2 * kFwdPartialFloats;
      const float wgt = __builtin_amdgcn_exp2f(ps[(size_t)BQ * D + r] - M);
      lt += ps[(size_t)BQ * D + BQ + r] * wgt;
#pragma unroll
      for (int c = 0; c < D / 2; c += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(ps + (size_t)r * D + c0 + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) osum[c + i] += x4[i] * wgt;
      }
    }
  }
  const int row = qi * BQ + r;
  if (row < N) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    bf16_t* orow = o + base + (size_t)row * D + c0;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4)
      store4(orow + c, osum[c] * inv, osum[c + 1] * inv, osum[c + 2] * inv, osum[c + 3] * inv);
    if ((tid & 1) == 0)
      lse[(size_t)bh * N + row] = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
  }
  if (tid == 0) done[entry] = 0;   // ready for the next call
}

// Forward for 64-row query blocks (two waves) with 32-key tiles: K and V
// double-buffered in 32 KB of LDS, so that four workgroups share a CU and
// each SIMD runs two waves (the 64-key tiles of fwd_async_kernel allow two
// such workgroups per CU, one wave per SIMD): 1.3B layer with 64 x 64
// blocks, 0.515 -> 0.433 ms.  Each list entry (a 64-key block) is walked as
// two 32-key steps.  With four-wave workgroups the same tiles gain 1.5% on
// the benchmark masks and lose 6% on a sink mask, so 128-row blocks keep the
// 64-key kernel.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 3)))
void fwd_async32_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                        const bf16_t* __restrict__ v, const int32_t* __restrict__ row_idx,
                        const int4* __restrict__ items, const int4* __restrict__ splits,
                        int* __restrict__ done, float* __restrict__ partials, int nrows, int N,
                        int Tq, int Tk, float scale_log2, bf16_t* __restrict__ o,
                        float* __restrict__ lse) {
  static_assert(NW == 2, "wave 0 copies K, wave 1 copies V");
  constexpr int D = 128;
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int TILE = 32 * D;
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) uint16_t kb0[TILE], kb1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[TILE], vb1[TILE];
  __shared__ int last_segment;

  const int4 item = items[blockIdx.x];
  int4 sp;
  if (!plan_item_ok(item, nrows, Tk, kRowPlan, splits, sp)) return;
  const int wg = item.x;
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const rsrc_t rk = make_rsrc(k + base, (uint32_t)N * D * 2);
  const rsrc_t rv = make_rsrc(v + base, (uint32_t)N * D * 2);
  uint32_t uo[4];
  unit_offsets(lane, uo);
  const SwzAddr addr0(lane);
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  bf16x8 qf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    qf[kk] = qvalid ? load8(q + base + (size_t)qrow * D + 16 * kk + 8 * h) : zero8();

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();
  float m = -INFINITY, lsum = 0.f;

  // half-steps u = 0 .. 2 cnt - 1: keys lst[u / 2] * 64 + 32 (u % 2)
  const int cnt = item.z, steps = 2 * cnt;
  const int32_t* lst = row_idx + (size_t)wg * Tk + item.y;
  auto key_at = [&](int u) { return u < steps ? lst[u >> 1] * 64 + 32 * (u & 1) : 0; };
  // wave 0 copies the 32 rows of K, wave 1 those of V
  auto copy_half = [&](int key0, uint16_t* kd, uint16_t* vd) {
    copy_groups<2>(w == 0 ? rk : rv, key0, 0, w == 0 ? kd : vd, uo);
  };
  int key_cur = key_at(0);
  if (steps > 0) copy_half(key_cur, kb0, vb0);
  int key_nxt = key_at(1);

  double_buffered(steps, [&](int u, auto parity) {
    constexpr bool odd = decltype(parity)::value == 1;
    const uint16_t* kt = odd ? kb1 : kb0;
    const uint16_t* vt = odd ? vb1 : vb0;
    const int key0 = key_cur;
    wait_vm_lgkm0<0>();
    __syncthreads();
    if (u + 1 < steps) copy_half(key_nxt, odd ? kb0 : kb1, odd ? vb0 : vb1);
    key_cur = key_nxt;
    key_nxt = key_at(u + 2);
    if (key0 >= N) return;   // the second half of a partial last block, all past N
    const SwzAddr A = addr0.fresh();

    f32x16 s = zero16();
    {
      bf16x8 ka[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) ka[kk] = rd_row(kt, A.row(0, kk));
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) s = mfma32(ka[kk], qf[kk], s);
    }
    if (key0 + 32 > N) {
      const int lim = N - key0 - 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) >= lim) s[e] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
    mx = wave_max32(mx) * scale_log2;
    if (__any(mx > m + kRescaleThreshold)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) acc[db] *= alpha;
    }
    bf16x8 va[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) va[db] = rd_tr(vt, A, 0, db);
    float ps = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], scale_log2, -m));
      pf[e >> 3][e & 7] = (__bf16)pv;
      ps += pv;
    }
    lsum += ps;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      bf16x8 vn[ND];
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        acc[db] = mfma32(va[db], pf[tt], acc[db]);
        if (tt < 1) vn[db] = rd_tr(vt, A, tt + 1, db);
      }
      if (tt < 1)
#pragma unroll
        for (int db = 0; db < ND; ++db) va[db] = vn[db];
    }
  });

  const float ltot = wave_sum32(lsum);
  if (item.w < 0) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    bf16_t* orow = o + base + (size_t)(qvalid ? qrow : 0) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) store_row32(orow + 32 * db, acc[db], inv, h, qvalid);
    if (qvalid && h == 0)
      lse[(size_t)bh * N + qrow] = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
    return;
  }
  // one segment of a split row: O^T rows, m and l into its partial slot
  // ([BQ rows][D] unnormalised O, then m[BQ], l[BQ])
  const int entry = item.w >> 10, seg = item.w & 1023;
  {
    const int r = w * 32 + l32;
    float* part = partials + (size_t)(sp.y + seg) * kFwdPartialFloats;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(part + (size_t)r * D + 32 * db + 8 * g + 4 * h, acc[db][4 * g],
               acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]);
    part[(size_t)BQ * D + (h == 0 ? r : BQ + r)] = h == 0 ? m : ltot;
  }
  // release the partial, count this segment done; the last one combines
  __threadfence();
  __syncthreads();
  if (tid == 0) last_segment = atomicAdd(&done[entry], 1) == sp.z - 1;
  __syncthreads();
  if (!last_segment) return;
  __threadfence();
  // two threads per row, each half of its D columns
  const int r = tid >> 1, c0 = (tid & 1) * (D / 2);
  const float* part0 = partials + (size_t)sp.y * kFwdPartialFloats;
  float M = -INFINITY;
  for (int s2 = 0; s2 < sp.z; ++s2)
    M = fmaxf(M, part0[(size_t)s2 * kFwdPartialFloats + (size_t)BQ * D + r]);
  float osum[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) osum[c] = 0.f;
  float lt = 0.f;
  if (M > -INFINITY) {
    for (int s2 = 0; s2 < sp.z; ++s2) {
      const float* ps = part0 + (size_t)s2 * kFwdPartialFloats;
      const float wgt = __builtin_amdgcn_exp2f(ps[(size_t)BQ * D + r] - M);
      lt += ps[(size_t)BQ * D + BQ + r] * wgt;
#pragma unroll
      for (int c = 0; c < D / 2; c += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(ps + (size_t)r * D + c0 + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) osum[c + i] += x4[i] * wgt;
      }
    }
  }
  const int row = qi * BQ + r;
  if (row < N) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    bf16_t* orow = o + base + (size_t)row * D + c0;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4)
      store4(orow + c, osum[c] * inv, osum[c + 1] * inv, osum[c + 2] * inv, osum[c + 3] * inv);
    if ((tid & 1) == 0)
      lse[(size_t)bh * N + row] = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
  }
  if (tid == 0) done[entry] = 0;   // ready for the next call
}


// dQ for bf16 and d = 128 with the same K and V rings as the forward, one
// workgroup per item of the row plan.  A segment of a split row leaves its
// fp32 dQ^T rows in a partial slot; the last segment adds the slots in
// segment order.  Every segment forms Delta and the LSE of its rows; the
// first (or the whole row) leaves them in the workspace for dK/dV.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1, 2)))
void dq_async_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ o,
                     const bf16_t* __restrict__ dout, const float* __restrict__ lse,
                     float* __restrict__ stats, const int32_t* __restrict__ row_idx,
                     const int4* __restrict__ items, const int4* __restrict__ splits,
                     int* __restrict__ done, float* __restrict__ partials, int nrows, int N,
                     int Tq, int Tk, float scale_log2, float scale, bf16_t* __restrict__ dq) {
  constexpr int D = 128;
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int TILE = 64 * D;
  constexpr int KCOPIES = 16 / NW;   // copy instructions per wave per tile tensor
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) uint16_t kb0[TILE], kb1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[TILE], vb1[TILE];
  __shared__ int last_segment;

  const int4 item = items[blockIdx.x];
  int4 sp;
  if (!plan_item_ok(item, nrows, Tk, kRowPlan, splits, sp)) return;
  const int wg = item.x;
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const rsrc_t rk = make_rsrc(k + base, (uint32_t)N * D * 2);
  const rsrc_t rv = make_rsrc(v + base, (uint32_t)N * D * 2);
  uint32_t uo[4];
  unit_offsets(lane, uo);
  const SwzAddr addr0(lane);
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  // the first tiles' copies go out before the row loads below
  const int cnt = item.z;
  const int32_t* lst = row_idx + (size_t)wg * Tk + item.y;
  auto key_at = [&](int t) { return t < cnt ? lst[t] * 64 : 0; };
  int key_t = key_at(0), key_t1 = key_at(1);
  if (cnt > 0) {
    copy_groups<KCOPIES / 4>(rk, key_t, w * KCOPIES, kb0, uo);
    copy_groups<KCOPIES / 4>(rv, key_t, w * KCOPIES, vb0, uo);
  }

  bf16x8 qf[NK], df[NK];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const size_t off = base + (size_t)qrow * D + 16 * kk + 8 * h;
    qf[kk] = qvalid ? load8(q + off) : zero8();
    df[kk] = qvalid ? load8(dout + off) : zero8();
    if (qvalid) dpart += delta_part(o + off, df[kk]);
  }
  // Delta = rowsum(dO * O): the two half-waves hold alternate 8-wide pieces
  // of the row.  Both statistics of every row of the block, padding rows
  // (zeros) included, are kept for the dK/dV kernel.
  const float dl = wave_sum32(dpart);
  // The dP accumulators start at -Delta, so that the MFMAs leave dP - Delta
  // (the row's Delta is the same for all of a lane's elements): 32 fewer
  // vector subtractions per 64-key step.
  f32x16 neg_dl;
#pragma unroll
  for (int e = 0; e < 16; ++e) neg_dl[e] = -dl;
  const float l2 = qvalid ? lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  if (item.w < 0 || (item.w & 1023) == 0)
    stats[stat_lse2(bh, stat_groups(N), qrow) + 32 * h] = h ? dl : l2;

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();

  double_buffered(cnt, [&](int t, auto parity) {
    constexpr bool odd = decltype(parity)::value == 1;
    const uint16_t* kt = odd ? kb1 : kb0;
    const uint16_t* vt = odd ? vb1 : vb0;
    const int key0 = key_t;
    wait_vm_lgkm0<0>();
    __syncthreads();
    if (t + 1 < cnt) copy_kv_tile<NW>(rk, rv, key_t1, odd ? kb0 : kb1, odd ? vb0 : vb1, w, uo);
    key_t = key_t1;
    key_t1 = key_at(t + 2);
    const SwzAddr A = addr0.fresh();

    // the two 32-key halves one after the other, so that only one half's S
    // and dP are live at a time
    const bool tail = key0 + 64 > N;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 sb = zero16(), dpb = neg_dl;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        sb = mfma32(rd_row(kt, A.row(b, kk)), qf[kk], sb);
        dpb = mfma32(rd_row(vt, A.row(b, kk)), df[kk], dpb);
      }
      // dS = P * (dP - Delta)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e], scale_log2, -l2));
        sb[e] = pv * dpb[e];
      }
      if (tail) {  // keys past N (zero rows) enter the dQ contraction: zero their dS
        const int lim = N - key0 - 4 * h;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + 8 * (e >> 2) + (e & 3) >= lim) sb[e] = 0.f;
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 sf = pack8(sb, 8 * t2);
#pragma unroll
        for (int db = 0; db < ND; ++db)
          acc[db] = mfma32(rd_tr(kt, A, 2 * b + t2, db), sf, acc[db]);
      }
    }
  });

  if (item.w < 0) {
    bf16_t* row = dq + base + (size_t)(qvalid ? qrow : 0) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) store_row32(row + 32 * db, acc[db], scale, h, qvalid);
    return;
  }
  // one segment of a split row: fp32 dQ^T rows into its partial slot
  const int entry = item.w >> 10, seg = item.w & 1023;
  {
    const int r = w * 32 + l32;
    float* part = partials + (size_t)(sp.y + seg) * kDqPartialFloats + (size_t)r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(part + 32 * db + 8 * g + 4 * h, acc[db][4 * g], acc[db][4 * g + 1],
               acc[db][4 * g + 2], acc[db][4 * g + 3]);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) last_segment = atomicAdd(&done[entry], 1) == sp.z - 1;
  __syncthreads();
  if (!last_segment) return;
  __threadfence();
  // two threads per row, each half of its D columns, segments in order
  const int r = tid >> 1, c0 = (tid & 1) * (D / 2);
  const float* part0 = partials + (size_t)sp.y * kDqPartialFloats + (size_t)r * D + c0;
  float gsum[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) gsum[c] = 0.f;
  for (int s2 = 0; s2 < sp.z; ++s2) {
    const float* ps = part0 + (size_t)s2 * kDqPartialFloats;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(ps + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) gsum[c + i] += x4[i];
    }
  }
  const int row = qi * BQ + r;
  if (row < N) {
    bf16_t* grow = dq + base + (size_t)row * D + c0;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4)
      store4(grow + c, gsum[c] * scale, gsum[c + 1] * scale, gsum[c + 2] * scale,
             gsum[c + 3] * scale);
  }
  if (tid == 0) done[entry] = 0;   // ready for the next call
}

// dQ for 64-row query blocks with 32-key tiles (K and V double-buffered in
// 32 KB of LDS), so that four two-wave workgroups share a CU instead of two:
// 1.3B layer with 64 x 64 blocks, 0.714 -> 0.575 ms.  Otherwise as
// dq_async_kernel.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 3)))
void dq_async32_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                       const bf16_t* __restrict__ v, const bf16_t* __restrict__ o,
                       const bf16_t* __restrict__ dout, const float* __restrict__ lse,
                       float* __restrict__ stats, const int32_t* __restrict__ row_idx,
                       const int4* __restrict__ items, const int4* __restrict__ splits,
                       int* __restrict__ done, float* __restrict__ partials, int nrows, int N,
                       int Tq, int Tk, float scale_log2, float scale, bf16_t* __restrict__ dq) {
  static_assert(NW == 2, "wave 0 copies K, wave 1 copies V");
  constexpr int D = 128;
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int TILE = 32 * D;
  constexpr int BQ = NW * 32;
  __shared__ __attribute__((aligned(16))) uint16_t kb0[TILE], kb1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[TILE], vb1[TILE];
  __shared__ int last_segment;

  const int4 item = items[blockIdx.x];
  int4 sp;
  if (!plan_item_ok(item, nrows, Tk, kRowPlan, splits, sp)) return;
  const int wg = item.x;
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const rsrc_t rk = make_rsrc(k + base, (uint32_t)N * D * 2);
  const rsrc_t rv = make_rsrc(v + base, (uint32_t)N * D * 2);
  uint32_t uo[4];
  unit_offsets(lane, uo);
  const SwzAddr addr0(lane);
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  // half-steps u = 0 .. 2 cnt - 1: keys lst[u / 2] * 64 + 32 (u % 2)
  const int cnt = item.z, steps = 2 * cnt;
  const int32_t* lst = row_idx + (size_t)wg * Tk + item.y;
  auto key_at = [&](int u) { return u < steps ? lst[u >> 1] * 64 + 32 * (u & 1) : 0; };
  auto copy_half = [&](int key0, uint16_t* kd, uint16_t* vd) {
    copy_groups<2>(w == 0 ? rk : rv, key0, 0, w == 0 ? kd : vd, uo);
  };
  int key_cur = key_at(0), key_nxt = key_at(1);
  if (steps > 0) copy_half(key_cur, kb0, vb0);

  bf16x8 qf[NK], df[NK];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const size_t off = base + (size_t)qrow * D + 16 * kk + 8 * h;
    qf[kk] = qvalid ? load8(q + off) : zero8();
    df[kk] = qvalid ? load8(dout + off) : zero8();
    if (qvalid) dpart += delta_part(o + off, df[kk]);
  }
  const float dl = wave_sum32(dpart);
  // The dP accumulators start at -Delta, so that the MFMAs leave dP - Delta
  // (the row's Delta is the same for all of a lane's elements): 32 fewer
  // vector subtractions per 64-key step.
  f32x16 neg_dl;
#pragma unroll
  for (int e = 0; e < 16; ++e) neg_dl[e] = -dl;
  const float l2 = qvalid ? lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  if (item.w < 0 || (item.w & 1023) == 0)
    stats[stat_lse2(bh, stat_groups(N), qrow) + 32 * h] = h ? dl : l2;

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();

  double_buffered(steps, [&](int u, auto parity) {
    constexpr bool odd = decltype(parity)::value == 1;
    const uint16_t* kt = odd ? kb1 : kb0;
    const uint16_t* vt = odd ? vb1 : vb0;
    const int key0 = key_cur;
    wait_vm_lgkm0<0>();
    __syncthreads();
    if (u + 1 < steps) copy_half(key_nxt, odd ? kb0 : kb1, odd ? vb0 : vb1);
    key_cur = key_nxt;
    key_nxt = key_at(u + 2);
    if (key0 >= N) return;   // the second half of a partial last block, all past N
    const SwzAddr A = addr0.fresh();
    f32x16 sb = zero16(), dpb = neg_dl;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      sb = mfma32(rd_row(kt, A.row(0, kk)), qf[kk], sb);
      dpb = mfma32(rd_row(vt, A.row(0, kk)), df[kk], dpb);
    }
    // dS = P * (dP - Delta)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e], scale_log2, -l2));
      sb[e] = pv * dpb[e];
    }
    if (key0 + 32 > N) {  // keys past N (zero rows) enter the dQ contraction: zero their dS
      const int lim = N - key0 - 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) >= lim) sb[e] = 0.f;
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const bf16x8 sf = pack8(sb, 8 * t2);
#pragma unroll
      for (int db = 0; db < ND; ++db) acc[db] = mfma32(rd_tr(kt, A, t2, db), sf, acc[db]);
    }
  });

  if (item.w < 0) {
    bf16_t* row = dq + base + (size_t)(qvalid ? qrow : 0) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) store_row32(row + 32 * db, acc[db], scale, h, qvalid);
    return;
  }
  // one segment of a split row: fp32 dQ^T rows into its partial slot
  const int entry = item.w >> 10, seg = item.w & 1023;
  {
    const int r = w * 32 + l32;
    float* part = partials + (size_t)(sp.y + seg) * kDqPartialFloats + (size_t)r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(part + 32 * db + 8 * g + 4 * h, acc[db][4 * g], acc[db][4 * g + 1],
               acc[db][4 * g + 2], acc[db][4 * g + 3]);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) last_segment = atomicAdd(&done[entry], 1) == sp.z - 1;
  __syncthreads();
  if (!last_segment) return;
  __threadfence();
  // two threads per row, each half of its D columns, segments in order
  const int r = tid >> 1, c0 = (tid & 1) * (D / 2);
  const float* part0 = partials + (size_t)sp.y * kDqPartialFloats + (size_t)r * D + c0;
  float gsum[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) gsum[c] = 0.f;
  for (int s2 = 0; s2 < sp.z; ++s2) {
    const float* ps = part0 + (size_t)s2 * kDqPartialFloats;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(ps + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) gsum[c + i] += x4[i];
    }
  }
  const int row = qi * BQ + r;
  if (row < N) {
    bf16_t* grow = dq + base + (size_t)row * D + c0;
#pragma unroll
    for (int c = 0; c < D / 2; c += 4)
      store4(grow + c, gsum[c] * scale, gsum[c + 1] * scale, gsum[c + 2] * scale,
             gsum[c + 3] * scale);
  }
  if (tid == 0) done[entry] = 0;   // ready for the next call
}


// ---------------------------------------------------------------------------
// Backward dK, dV: one workgroup (4 waves) per key block of 64 keys.
//
// Waves form two pairs.  Pair p walks the 32-row slices 2j + p of every
// query block in the key block's column list; in a pair, wave kb accumulates
// dK and dV of keys key0 + 32kb .. +31 over all of d (the two pairs' partial
// sums are added at the end).  The two waves of a pair stage a slice
// together (wave 0 loads Q, wave 1 loads dO; each keeps its own half as MFMA
// A operands and reads the other half from LDS).  Both pairs step in lock
// step: one workgroup barrier after staging, one before the slice buffers
// are overwritten.
// ---------------------------------------------------------------------------
template <typename T, int D, int BQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const T* __restrict__ dout, const float* __restrict__ stats,
                 const int32_t* __restrict__ col_cnt,
                 const int32_t* __restrict__ col_idx, int N,
                 int Tq, int Tk, float scale_log2, float scale, T* __restrict__ dk,
                 T* __restrict__ dv) {
  constexpr int NT = 256;
  using KT = Tile<D, kRows>;   // K, V tiles: fragment reads
  using ST = Tile<D, kBoth>;   // Q / dO slices: fragment and transposed reads
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int CPT = 64 * (D / 8) / NT;
  constexpr int SUB = BQ / 32;   // 32-row slices per query block
  constexpr int SPP = SUB / 2;   // slices per pair per query block
  constexpr int RS = D + 4;      // fp32 staging of a wave's output tile
  constexpr int TILE_BYTES = 2 * 64 * KT::kRowElems * 2;
  constexpr int SLICE_BYTES = 2 * 2 * 32 * ST::kRowElems * 2;
  constexpr int STAGE_BYTES = 2 * 2 * 32 * RS * 4;  // [key half][dV | dK] fp32 tiles
  constexpr int SMEM_BYTES = TILE_BYTES + SLICE_BYTES > STAGE_BYTES ? TILE_BYTES + SLICE_BYTES
                                                                    : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) float st[2][2][32];  // [pair][lse2 | Delta][row]

  uint16_t* k_lds = reinterpret_cast<uint16_t*>(smem);
  uint16_t* v_lds = k_lds + 64 * KT::kRowElems;
  uint16_t* slices = v_lds + 64 * KT::kRowElems;               // [pair][Q | dO][32 rows]

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / Tk, kj = wg % Tk;
  const int key0 = kj * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int pair = w >> 1, kb = w & 1;
  const size_t base = (size_t)bh * N * D;

  {
    bf16x8 r[CPT];
    fetch_tile<T, D, NT>(k + base, key0, N, tid, r);
    put_tile<D, kRows, NT>(k_lds, tid, r);
    fetch_tile<T, D, NT>(v + base, key0, N, tid, r);
    put_tile<D, kRows, NT>(v_lds, tid, r);
  }
  // the tiles are complete before any wave reads them, and before the output
  // staging (which reuses this memory) of a key block with an empty list
  __syncthreads();

  uint16_t* sq = slices + (2 * pair) * 32 * ST::kRowElems;   // this pair's Q slice
  uint16_t* sd = sq + 32 * ST::kRowElems;                     // this pair's dO slice
  uint16_t* mine = kb == 0 ? sq : sd;              // the half this wave stages
  const T* src = kb == 0 ? q : dout;
  const int G = stat_groups(N);
  const int krow = 32 * kb + l32;                  // this lane's row of K, V

  f32x16 accv[ND], acck[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    accv[db] = zero16();
    acck[db] = zero16();
  }

  const int cnt = list_len(col_cnt[wg], Tq);
  const int32_t* lst = col_idx + (size_t)wg * Tq;
  const int steps = cnt * SPP;

  // own[kk]: row l32 of this wave's half of the slice, d = 16kk + 8h .. +7
  bf16x8 own[NK];
  float stat = 0.f;
  auto fetch = [&](int s) {
    const int row = lst[s / SPP] * BQ + 32 * (2 * (s % SPP) + pair) + l32;
    const bool ok = (unsigned)row < (unsigned)N;
    const T* p = src + base + (size_t)row * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) own[kk] = ok ? load8(p + 16 * kk) : zero8();
    // wave 0: log2-scaled LSE (+inf on padding rows: P = 0); wave 1: Delta
    const float x = ok ? stats[stat_lse2(bh, G, row) + 32 * kb] : 0.f;
    stat = kb == 0 ? (ok ? x : INFINITY) : x;
  };

  if (steps > 0) fetch(0);
  for (int s = 0; s < steps; ++s) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      *reinterpret_cast<bf16x8*>(mine + ST::off(l32, 16 * kk + 8 * h)) = own[kk];
    if (h == 0) st[pair][kb][l32] = stat;
    __syncthreads();
    // S = Q K^T and dP = dO V^T: the slice's 32 rows against this wave's 32 keys
    f32x16 sa = zero16(), dpa = zero16();
    if (kb == 0) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int c = 16 * kk + 8 * h;
        sa = mfma32(own[kk], lds_read8(k_lds + KT::off(krow, c)), sa);
        dpa = mfma32(lds_read8(sd + ST::off(l32, c)), lds_read8(v_lds + KT::off(krow, c)), dpa);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int c = 16 * kk + 8 * h;
        sa = mfma32(lds_read8(sq + ST::off(l32, c)), lds_read8(k_lds + KT::off(krow, c)), sa);
        dpa = mfma32(own[kk], lds_read8(v_lds + KT::off(krow, c)), dpa);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < steps) fetch(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    // P = exp(S/sqrt(d) - LSE) and dS = P * (dP - Delta) for rows 8g+4h+i,
    // packed at once into the B operands of the two 16-row steps.  Keys past
    // N need no mask: their K and V rows are zero and they only feed their
    // own (unstored) dK, dV rows.
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 L = *reinterpret_cast<const f32x4*>(&st[pair][0][8 * g + 4 * h]);
      const f32x4 Dl = *reinterpret_cast<const f32x4*>(&st[pair][1][8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g + i;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], scale_log2, -L[i]));
        pb[g >> 1][4 * (g & 1) + i] = (__bf16)pv;
        sb[g >> 1][4 * (g & 1) + i] = (__bf16)(pv * (dpa[e] - Dl[i]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the slice's rows
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        accv[db] = mfma32(tr_operand<D, kBoth>(sd, 16 * t, 32 * db, lane), pb[t], accv[db]);
        acck[db] = mfma32(tr_operand<D, kBoth>(sq, 16 * t, 32 * db, lane), sb[t], acck[db]);
      }
    __syncthreads();
  }

  // The two waves of a key half (one per pair) hold partial sums over
  // different slices.  Pair 1 hands its tiles to pair 0 through LDS; pair 0
  // adds them (always in this order) and stores.  Accumulator element e of
  // block db is d = 32db + 8(e/4) + 4h + e%4 at key 32kb + l32; the sum goes
  // back to LDS so that the stores are whole 4-element runs of a key's row.
  float* tile[2];
#pragma unroll
  for (int which = 0; which < 2; ++which)
    tile[which] = reinterpret_cast<float*>(smem) + (kb * 2 + which) * 32 * RS;
  if (pair == 1) {
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          tile[which][l32 * RS + 32 * db + 8 * (e >> 2) + 4 * h + (e & 3)] =
              which == 0 ? accv[db][e] : acck[db][e];
  }
  __syncthreads();
  if (pair == 0) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const float mul = which == 0 ? 1.f : scale;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float* p = tile[which] + l32 * RS + 32 * db + 8 * (e >> 2) + 4 * h + (e & 3);
          *p = ((which == 0 ? accv[db][e] : acck[db][e]) + *p) * mul;
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      T* out = (which == 0 ? dv : dk) + base;
      for (int ch = lane; ch < 32 * D / 4; ch += 64) {
        const int r = ch / (D / 4), c4 = (ch % (D / 4)) * 4;
        const int key = key0 + 32 * kb + r;
        if (key < N) {
          const float* p = tile[which] + r * RS + c4;
          store4(out + (size_t)key * D + c4, p[0], p[1], p[2], p[3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward dK, dV for bf16 and d = 128: one workgroup of two waves per key
// block.
//
// Wave kb owns keys key0 + 32kb .. +31: their K and V fragments (the B
// operands of S = Q K^T and dP = dO V^T) live in registers for the whole
// kernel, their dK^T and dV^T tiles (32 x 128 each) in accumulators.  Both
// waves walk every 32-row slice of the query blocks in the column list; each
// slice's Q rows and statistics (copied by wave 0) and dO rows (wave 1) go
// straight to an LDS double buffer (see copy_groups, double_buffered) that
// the two waves share, so the only barrier is between the two.  Four
// workgroups share a CU, so the two waves on a SIMD belong to different
// workgroups and overlap their phases freely.
// ---------------------------------------------------------------------------
//
// With DQ set (the fused variant, sa2_attn_bwd_atomic_dq), each step also
// forms dQ^T of the slice's rows over this block's 64 keys, dQ^T = K^T dS^T,
// and adds it to the fp32 accumulator dq_acc with vector atomics: K is kept
// in LDS for the transposed operand, and dS goes through LDS to be read one
// row per lane.  The order of those additions is not fixed.
template <int BQ, bool DQ>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_pair_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                      const float* __restrict__ stats, const int4* __restrict__ items,
                      const int32_t* __restrict__ col_idx, int N, int Tq, int Tk,
                      float scale_log2, float scale, bf16_t* __restrict__ dk,
                      bf16_t* __restrict__ dv, const int4* __restrict__ splits,
                      int* __restrict__ done, float* __restrict__ partials, int ncols,
                      float* __restrict__ dq_acc) {
  constexpr int D = 128;
  using ST = Tile<D, kBoth>;   // slices: permuted, unpadded rows of 256 bytes
  static_assert(ST::kSwizzled, "slices are copied as whole 256-byte rows");
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int SUB = BQ / 32;   // slices per query block
  constexpr int SLICE = 32 * D;  // elements of one slice tensor
  __shared__ __attribute__((aligned(16))) uint16_t sq0[SLICE], sq1[SLICE];   // Q slices
  __shared__ __attribute__((aligned(16))) uint16_t so0[SLICE], so1[SLICE];   // dO slices
  __shared__ __attribute__((aligned(16))) float st0[64], st1[64];            // [lse | Delta]
  __shared__ int last_segment;
  // fused variant only: the K tile (64 keys, permuted rows) and dS [32 rows][64 keys]
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[DQ ? 64 * D : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[DQ ? 32 * 64 : 8];

  // {block, first list entry, entries, -1 or split entry * 1024 + segment};
  // an entry that does not fit this call (a plan written for another mask,
  // or never written) is skipped, so nothing is read or written out of range
  const int4 item = items[blockIdx.x];
  int4 sp;   // {block, first partial slot, segments}
  if (!plan_item_ok(item, ncols, Tq, kColPlan, splits, sp)) return;
  const int wg = item.x;
  const int bh = wg / Tk, kj = wg % Tk;
  const int key0 = kj * 64;
  const int tid = threadIdx.x, lane = tid & 63, kb = uniform(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;

  // K and V fragments of this wave's keys, zero past N.  Without the fused
  // dQ, the K rows and then the V rows are copied whole into this wave's
  // second slice buffer (free until step 0 issues its copy) and read from
  // there once the first slice's copy is out.
  uint32_t uo[4];
  unit_offsets(lane, uo);
  uint16_t* kst = kb == 0 ? sq1 : so1;
  if constexpr (!DQ)
    copy_groups<2>(make_rsrc(k + base, (uint32_t)N * D * 2), key0 + 32 * kb, 0, kst, uo);
  bf16x8 kf[NK], vf[NK];
  {
    const int key = key0 + 32 * kb + l32;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const size_t off = base + (size_t)key * D + 16 * kk + 8 * h;
      if constexpr (DQ) {
        kf[kk] = key < N ? load8(k + off) : zero8();
        vf[kk] = key < N ? load8(v + off) : zero8();
      }
    }
  }

  const int cnt = item.z;
  const int32_t* lst = col_idx + (size_t)wg * Tq + item.y;
  const int steps = cnt * SUB;
  // wave 0 copies Q and the statistics, wave 1 copies dO; rows past N arrive
  // as zeros, their statistics as the dQ kernel wrote them (zeros)
  const rsrc_t rsrc = make_rsrc((kb == 0 ? q : dout) + base, (uint32_t)N * D * 2);
  const int G = stat_groups(N);
  const rsrc_t rst = make_rsrc(stats + (size_t)bh * G * 64, (uint32_t)G * 256);
  auto slice_row = [&](int s) { return s < steps ? lst[s / SUB] * BQ + 32 * (s % SUB) : 0; };
  auto copy = [&](int row0, uint16_t* dq_, uint16_t* do_, float* ds_) {
    if (kb == 0) {
      copy_groups<2>(rsrc, row0, 0, dq_, uo);
      buf_lds4<0>(rst, ds_, 4 * lane, (uint32_t)row0 * 8u);
    } else {
      copy_groups<2>(rsrc, row0, 0, do_, uo);
    }
  };

  f32x16 accv[ND], acck[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    accv[db] = zero16();
    acck[db] = zero16();
  }

  const SwzAddr addr0(lane);

  if constexpr (DQ) {   // the K tile, eight groups of four rows per wave (waited at step 0)
    if (steps > 0) copy_groups<2>(make_rsrc(k + base, (uint32_t)N * D * 2), key0, 8 * kb, k_lds, uo);
  }
  int row_cur = slice_row(0);
  if (steps > 0) copy(row_cur, sq0, so0, st0);
  int row_nxt = slice_row(1);
  if constexpr (!DQ) {
    // the K copy went out before the first slice's (at least 8) copy instructions
    if (steps > 0) wait_vm_lgkm0<8>();
    else wait_vm_lgkm0<0>();
    wave_lds_sync();
    const SwzAddr ka(lane);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kf[kk] = rd_row(kst, ka.row(0, kk));
    // then the V rows through the same buffer, once the K reads are done
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    copy_groups<2>(make_rsrc(v + base, (uint32_t)N * D * 2), key0 + 32 * kb, 0, kst, uo);
    wait_vm_lgkm0<0>();
    wave_lds_sync();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) vf[kk] = rd_row(kst, ka.row(0, kk));
  }
  double_buffered(steps, [&](int s, auto parity) {
    constexpr bool odd = decltype(parity)::value == 1;
    const uint16_t* sq = odd ? sq1 : sq0;
    const uint16_t* so = odd ? so1 : so0;
    const float* stl = odd ? st1 : st0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 1 < steps) copy(row_nxt, odd ? sq0 : sq1, odd ? so0 : so1, odd ? st0 : st1);
    const int row0 = row_cur;
    row_cur = row_nxt;
    row_nxt = slice_row(s + 2);
    const SwzAddr A = addr0.fresh();

    // S = Q K^T and dP = dO V^T for the slice's 32 rows and this wave's keys,
    // the row fragments of step kk read two steps ahead
    f32x16 sa = zero16(), dpa = zero16();
    {
      bf16x8 qa[NK], oa[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        qa[kk] = rd_row(sq, A.row(0, kk));
        oa[kk] = rd_row(so, A.row(0, kk));
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        sa = mfma32(qa[kk], kf[kk], sa);
        dpa = mfma32(oa[kk], vf[kk], dpa);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // reads of steps 0, 1
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMAs of step kk
        if (kk + 2 < NK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads of kk + 2
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // P and dS for rows 8g+4h+i, packed into the B operands of the two
    // 16-row steps.  No mask is needed: keys past N only feed their own,
    // unstored, dK and dV rows; query rows past N arrive as zero Q and dO
    // rows with zero statistics, so their P is exactly 1, their dS exactly 0,
    // and both meet zero rows in the dV and dK products.
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const f32x4 L = *reinterpret_cast<const f32x4*>(stl + 8 * gg + 4 * h);
      const f32x4 Dl = *reinterpret_cast<const f32x4*>(stl + 32 + 8 * gg + 4 * h);
      const int t = gg >> 1, o = 4 * (gg & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * gg + i;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], scale_log2, -L[i]));
        pb[t][o + i] = (__bf16)pv;
        sb[t][o + i] = (__bf16)(pv * (dpa[e] - Dl[i]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the slice's rows; the
    // transposed operands of a (t, db) step are read two steps ahead (in a
    // scheduling region of their own, so that the reads are not hoisted into
    // the S and dP phase, where their registers are taken)
    __builtin_amdgcn_sched_barrier(0);
    {
      bf16x8 ot[2 * ND], qt[2 * ND];
#pragma unroll
      for (int g = 0; g < 2 * ND; ++g) {
        ot[g] = rd_tr(so, A, g / ND, g % ND);
        qt[g] = rd_tr(sq, A, g / ND, g % ND);
      }
#pragma unroll
      for (int g = 0; g < 2 * ND; ++g) {
        accv[g % ND] = mfma32(ot[g], pb[g / ND], accv[g % ND]);
        acck[g % ND] = mfma32(qt[g], sb[g / ND], acck[g % ND]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // DS reads of steps 0, 1
#pragma unroll
      for (int g = 0; g < 2 * ND; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMAs of step g
        if (g + 2 < 2 * ND) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // reads of g + 2
      }
    }
    if constexpr (DQ) {
      // dS of rows 8gg + 4h + i at this lane's key, into [row][key] LDS
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8& sv = sb[gg >> 1];
          reinterpret_cast<__bf16*>(ds_lds)[(8 * gg + 4 * h + i) * 64 + 32 * kb + l32] =
              sv[4 * (gg & 1) + i];
        }
      __syncthreads();
      // dQ (rows x d) over the 64 keys: wave kb takes d = 64kb .. 64kb + 63.
      // The A operand dS takes this lane's row from ds_lds at the keys of
      // k-slots 8h + i <-> 16t + 8(i/4) + 4h + i%4; the B operand K (keys x
      // d) comes from the K tile by transposed reads with the same slots.
      // Lanes run along d, so each atomic instruction covers two rows of 32
      // consecutive floats.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int db = 2 * kb + j;
        f32x16 acc = zero16();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint16_t* r = ds_lds + l32 * 64 + 16 * t + 4 * h;
          const bf16x8 aop = cat(*reinterpret_cast<const bf16x4*>(r),
                                 *reinterpret_cast<const bf16x4*>(r + 8));
          acc = mfma32(aop, rd_tr(k_lds, A, t, db), acc);
        }
        // element e: row row0 + 8(e/4) + 4h + e%4, d = 32db + l32
        float* dst = dq_acc + base + (size_t)row0 * D + 32 * db + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 8 * (e >> 2) + 4 * h + (e & 3);
          if (row0 + r < N) unsafeAtomicAdd(dst + (size_t)r * D, acc[e]);
        }
      }
    }
  });

  // Element e of block db is d = 32db + 8(e/4) + 4h + e%4 at key 32kb + l32:
  // runs of four consecutive d of one key row.
  const int key = key0 + 32 * kb + l32;
  if (item.w >= 0) {
    // one segment of a split list: fp32 partial [dV | dK] rows of all 64 keys
    const int entry = item.w >> 10;
    float* pv = partials + (size_t)(sp.y + (item.w & 1023)) * kPartialFloats +
                (size_t)(32 * kb + l32) * D;
    float* pk = pv + 64 * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * db + 8 * g + 4 * h, e = 4 * g;
        store4(pv + c, accv[db][e], accv[db][e + 1], accv[db][e + 2], accv[db][e + 3]);
        store4(pk + c, acck[db][e] * scale, acck[db][e + 1] * scale, acck[db][e + 2] * scale,
               acck[db][e + 3] * scale);
      }
    // release the partial, count this segment done; the last one sums
    __threadfence();
    __syncthreads();
    if (tid == 0) last_segment = atomicAdd(&done[entry], 1) == sp.z - 1;
    __syncthreads();
    if (last_segment) {
      __threadfence();
      // thread t sums 16-byte groups t + 128j of the partials, all 32 of a
      // segment loaded at once, the segments in order
      constexpr int PER = (int)kPartialFloats / 4 / 128;
      const float* part = partials + (size_t)sp.y * kPartialFloats + 4 * tid;
      f32x4 acc[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] = *reinterpret_cast<const f32x4*>(part + 512 * j);
      for (int s2 = 1; s2 < sp.z; ++s2) {
        const float* ps = part + (size_t)s2 * kPartialFloats;
        f32x4 t[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) t[j] = *reinterpret_cast<const f32x4*>(ps + 512 * j);
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += t[j];
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int g = tid + 128 * j;
        const int r = (g / (D / 4)) % 64, c4 = (g % (D / 4)) * 4;   // dV rows, then dK rows
        if (key0 + r < N)
          store4((g < (int)kPartialFloats / 8 ? dv : dk) + base + (size_t)(key0 + r) * D + c4,
                 acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      }
      if (tid == 0) done[entry] = 0;   // ready for the next call
    }
  } else {
    const bool kv = key < N;
    bf16_t* rv = dv + base + (size_t)(kv ? key : 0) * D;
    bf16_t* rk = dk + base + (size_t)(kv ? key : 0) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      store_row32(rv + 32 * db, accv[db], 1.f, h, kv);
      store_row32(rk + 32 * db, acck[db], scale, h, kv);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused-variant helpers (bf16, d = 128).  dq_prep_kernel: per 128-row group
// of a head, Delta (from the bf16 dO that enters dP) and the base-2 LSE of
// every row into the statistics (zeros for padding rows), and the rows' fp32
// dQ accumulator zeroed; two threads per row, half of d each.
// dq_finish_kernel: dQ = accumulator / sqrt(d), rounded to bf16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void dq_prep_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                    const float* __restrict__ lse, float* __restrict__ stats,
                    float* __restrict__ dq_acc, int N, int G4) {
  constexpr int D = 128;
  const int bh = blockIdx.x / G4, grp = blockIdx.x % G4;
  const int tid = threadIdx.x, r = grp * 128 + (tid >> 1), half = tid & 1;
  const size_t base = (size_t)bh * N * D;
  float dpart = 0.f;
  if (r < N) {
    const size_t off = base + (size_t)r * D + 64 * half;
#pragma unroll
    for (int c = 0; c < 64; c += 8) dpart += delta_part(o + off + c, load8(dout + off + c));
    float* acc = dq_acc + off;
#pragma unroll
    for (int c = 0; c < 64; c += 4) store4(acc + c, 0.f, 0.f, 0.f, 0.f);
  }
  dpart += __shfl_xor(dpart, 1);
  if (half == 0) {
    const int G = stat_groups(N);
    stats[stat_delta(bh, G, r)] = r < N ? dpart : 0.f;
    stats[stat_lse2(bh, G, r)] = r < N ? lse[(size_t)bh * N + r] * kLog2e : 0.f;
  }
}

__global__ __launch_bounds__(256)
void dq_finish_kernel(const float* __restrict__ dq_acc, size_t n4, float scale,
                      bf16_t* __restrict__ dq) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(dq_acc + 4 * i);
    store4(dq + 4 * i, a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale);
  }
}

// ---------------------------------------------------------------------------
// Backward dQ: one workgroup per query block, walking its row list.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1, 2)))
void dq_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
               const T* __restrict__ o, const T* __restrict__ dout, const float* __restrict__ lse,
               float* __restrict__ stats, const int32_t* __restrict__ row_cnt,
               const int32_t* __restrict__ row_idx, int N,
               int Tq, int Tk, float scale_log2, float scale, T* __restrict__ dq) {
  constexpr int NT = NW * 64;
  using KT = Tile<D, kPad16>;  // K: fragment and transposed reads
  using VT = Tile<D, kRows>;   // V: fragment reads
  constexpr int NK = D / 16, ND = D / 32;
  constexpr int CPT = 64 * (D / 8) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[64 * KT::kRowElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[64 * VT::kRowElems];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / Tq, qi = wg % Tq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const size_t base = (size_t)bh * N * D;
  const T* kh = k + base;
  const T* vh = v + base;
  const int qrow = qi * (NW * 32) + w * 32 + l32;
  const bool qvalid = qrow < N;

  bf16x8 qf[NK], df[NK];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const size_t off = base + (size_t)qrow * D + 16 * kk + 8 * h;
    qf[kk] = qvalid ? load8(q + off) : zero8();
    df[kk] = qvalid ? load8(dout + off) : zero8();
    if (qvalid) dpart += delta_part(o + off, df[kk]);
  }
  // Delta = rowsum(dO * O): the two half-waves hold alternate 8-wide pieces
  // of the row.  It is kept for the dK/dV kernel.  Padding rows: dO = 0 and
  // Delta = 0 give dS = 0 whatever P is.
  const float dl = wave_sum32(dpart);
  const float l2 = qvalid ? lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  // both statistics of every row of the block, padding rows (zeros) included
  stats[stat_lse2(bh, stat_groups(N), qrow) + 32 * h] = h ? dl : l2;

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16();

  const int cnt = list_len(row_cnt[wg], Tk);
  const int32_t* lst = row_idx + (size_t)wg * Tk;
  bf16x8 kr[CPT], vr[CPT];
  if (cnt > 0) {
    fetch_tile<T, D, NT>(kh, lst[0] * 64, N, tid, kr);
    fetch_tile<T, D, NT>(vh, lst[0] * 64, N, tid, vr);
  }
  for (int t = 0; t < cnt; ++t) {
    const int key0 = lst[t] * 64;
    __syncthreads();
    put_tile<D, kPad16, NT>(k_lds, tid, kr);
    put_tile<D, kRows, NT>(v_lds, tid, vr);
    __syncthreads();
    if (t + 1 < cnt) {
      const int nk0 = lst[t + 1] * 64;
      fetch_tile<T, D, NT>(kh, nk0, N, tid, kr);
      fetch_tile<T, D, NT>(vh, nk0, N, tid, vr);
    }
    // the two 32-key halves one after the other, so that only one half's S
    // and dP are live at a time
    const bool tail = key0 + 64 > N;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 sb = zero16(), dpb = zero16();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int c = 16 * kk + 8 * h;
        sb = mfma32(lds_read8(k_lds + KT::off(32 * b + l32, c)), qf[kk], sb);
        dpb = mfma32(lds_read8(v_lds + VT::off(32 * b + l32, c)), df[kk], dpb);
      }
      // dS = P * (dP - Delta)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e], scale_log2, -l2));
        sb[e] = pv * (dpb[e] - dl);
      }
      if (tail) {  // keys past N enter the dQ contraction: zero them
        const int lim = N - key0 - 4 * h;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + 8 * (e >> 2) + (e & 3) >= lim) sb[e] = 0.f;
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const bf16x8 sf = pack8(sb, 8 * t2);
#pragma unroll
        for (int db = 0; db < ND; ++db)
          acc[db] = mfma32(tr_operand<D, kPad16>(k_lds, 32 * b + 16 * t2, 32 * db, lane), sf,
                           acc[db]);
      }
    }
  }
  if (qvalid) {
    T* row = dq + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(row + 32 * db + 8 * g + 4 * h, acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale,
               acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static sa2_status check_common(const char* fn, int dtype, int B, int H, int N, int d,
                               const sa2_mask* m) {
  if (!m) return fail(SA2_EINVAL, std::string(fn) + ": null mask");
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(SA2_EINVAL, std::string(fn) + ": B, H, N, d must be positive");
  if (dtype != SA2_BF16 && dtype != SA2_F32)
    return fail(SA2_EINVAL, std::string(fn) + ": unknown dtype");
  if (m->B != B || m->H != H || m->N != N || m->bq <= 0 || m->bk <= 0 ||
      m->Tq != cdiv(N, m->bq) || m->Tk != cdiv(N, m->bk))
    return fail(SA2_EINVAL, std::string(fn) + ": mask geometry does not match the call");
  if (d != 64 && d != 128) return fail(SA2_EUNSUPPORTED, std::string(fn) + ": d must be 64 or 128");
  if (m->bk != 64) return fail(SA2_EUNSUPPORTED, std::string(fn) + ": key blocks must be 64 tokens");
  if (m->bq != 64 && m->bq != 128)
    return fail(SA2_EUNSUPPORTED, std::string(fn) + ": query blocks must be 64 or 128 tokens");
  if ((size_t)B * H * m->Tq > 0x7fffffff || (size_t)B * H * m->Tk > 0x7fffffff)
    return fail(SA2_EUNSUPPORTED, std::string(fn) + ": too many blocks");
  return SA2_OK;
}

// A plan's pointers: from the mask's plan array (items, split entries, the
// completion counters of one kernel) and the partial slots of a workspace.
struct PlanPtrs {
  const int4 *items, *splits;
  int* done;
  float* partials;
};
static PlanPtrs plan_ptrs(int32_t* plan, int n, PlanKind kd, int ndone, int which,
                          float* partials) {
  const PlanLayout l = plan_layout(n, kd, ndone);
  char* b = reinterpret_cast<char*>(plan);
  return PlanPtrs{reinterpret_cast<const int4*>(b + l.items),
                  reinterpret_cast<const int4*>(b + l.splits),
                  reinterpret_cast<int*>(b + l.done) + (size_t)8 * kd.extra * which, partials};
}
static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
// Partial slots of a plan kind: 2 `extra` per XCD share.
static size_t partial_bytes(PlanKind kd, size_t floats) {
  return (size_t)8 * 2 * kd.extra * floats * sizeof(float);
}

template <typename T, int D, int NW>
static void launch_fwd(const void* q, const void* k, const void* v, const sa2_mask* m, int BH,
                       int N, float sl2, void* o, float* lse, hipStream_t s) {
  fwd_kernel<T, D, NW><<<BH * m->Tq, NW * 64, 0, s>>>(
      static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), m->row_cnt,
      m->row_idx, N, m->Tq, m->Tk, sl2, static_cast<T*>(o), lse);
}

template <int NW>
static void launch_fwd_async(const void* q, const void* k, const void* v, const sa2_mask* m,
                             int BH, int N, float sl2, void* o, float* lse, const PlanPtrs& rp,
                             hipStream_t s) {
  const int nrows = BH * m->Tq;
  if constexpr (NW == 2) {
    fwd_async32_kernel<NW><<<8 * plan_items_per_xcd(nrows, kRowPlan), NW * 64, 0, s>>>(
        static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
        static_cast<const bf16_t*>(v), m->row_idx, rp.items, rp.splits, rp.done, rp.partials,
        nrows, N, m->Tq, m->Tk, sl2, static_cast<bf16_t*>(o), lse);
    return;
  }
  fwd_async_kernel<NW><<<8 * plan_items_per_xcd(nrows, kRowPlan), NW * 64, 0, s>>>(
      static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
      static_cast<const bf16_t*>(v), m->row_idx, rp.items, rp.splits, rp.done, rp.partials,
      nrows, N, m->Tq, m->Tk, sl2, static_cast<bf16_t*>(o), lse);
}

template <typename T, int D>
static void dispatch_fwd(const void* q, const void* k, const void* v, const sa2_mask* m, int BH,
                         int N, float sl2, void* o, float* lse, const PlanPtrs& rp,
                         hipStream_t s) {
  if constexpr (D == 128 && sizeof(T) == 2) {
    if (m->bq == 128) launch_fwd_async<4>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
    else launch_fwd_async<2>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
    return;
  }
  if (m->bq == 128) launch_fwd<T, D, 4>(q, k, v, m, BH, N, sl2, o, lse, s);
  else launch_fwd<T, D, 2>(q, k, v, m, BH, N, sl2, o, lse, s);
}

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  const sa2_mask* m;
  int BH, N;
  float sl2, scale;
  void *dq, *dk, *dv;
  float* stats;
  PlanPtrs rows, cols;   // dQ and dK/dV plans (bf16, d = 128)
  hipStream_t s;
};

template <typename T, int D>
static void launch_dq(const BwdArgs& a) {
  const sa2_mask* m = a.m;
  if constexpr (D == 128 && sizeof(T) == 2) {
    const int nrows = a.BH * m->Tq;
#define SA2_DQ_ASYNC_ARGS                                                                     \
  static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),                            \
      static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.o),                        \
      static_cast<const bf16_t*>(a.dout), a.lse, a.stats, m->row_idx, a.rows.items,            \
      a.rows.splits, a.rows.done, a.rows.partials, nrows, a.N, m->Tq, m->Tk, a.sl2, a.scale,   \
      static_cast<bf16_t*>(a.dq)
    const int grid = 8 * plan_items_per_xcd(nrows, kRowPlan);
    if (m->bq == 128) dq_async_kernel<4><<<grid, 256, 0, a.s>>>(SA2_DQ_ASYNC_ARGS);
    else dq_async32_kernel<2><<<grid, 128, 0, a.s>>>(SA2_DQ_ASYNC_ARGS);
#undef SA2_DQ_ASYNC_ARGS
    return;
  }
#define SA2_DQ_ARGS                                                                          \
  static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),          \
      static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.lse, a.stats,              \
      m->row_cnt,                                                                             \
      m->row_idx, a.N, m->Tq, m->Tk, a.sl2, a.scale, static_cast<T*>(a.dq)
  if (m->bq == 128) dq_kernel<T, D, 4><<<a.BH * m->Tq, 256, 0, a.s>>>(SA2_DQ_ARGS);
  else dq_kernel<T, D, 2><<<a.BH * m->Tq, 128, 0, a.s>>>(SA2_DQ_ARGS);
#undef SA2_DQ_ARGS
}

template <typename T, int D>
static void launch_dkdv(const BwdArgs& a) {
  const sa2_mask* m = a.m;
  if constexpr (D == 128 && sizeof(T) == 2) {
    const int ncols = a.BH * m->Tk;
#define SA2_DKDV_PAIR_ARGS                                                                  \
  static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),                            \
      static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.dout), a.stats,             \
      a.cols.items, m->col_idx, a.N, m->Tq, m->Tk, a.sl2, a.scale,                             \
      static_cast<bf16_t*>(a.dk), static_cast<bf16_t*>(a.dv), a.cols.splits, a.cols.done,      \
      a.cols.partials, ncols
    const int grid = 8 * plan_items_per_xcd(ncols, kColPlan);
    if (m->bq == 128) dkdv_pair_kernel<128, false><<<grid, 128, 0, a.s>>>(SA2_DKDV_PAIR_ARGS, nullptr);
    else dkdv_pair_kernel<64, false><<<grid, 128, 0, a.s>>>(SA2_DKDV_PAIR_ARGS, nullptr);
#undef SA2_DKDV_PAIR_ARGS
    return;
  }
#define SA2_DKDV_ARGS                                                                         \
  static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),          \
      static_cast<const T*>(a.dout), a.stats, m->col_cnt, m->col_idx, a.N,          \
      m->Tq, m->Tk, a.sl2, a.scale, static_cast<T*>(a.dk), static_cast<T*>(a.dv)
  if (m->bq == 128) dkdv_kernel<T, D, 128><<<a.BH * m->Tk, 256, 0, a.s>>>(SA2_DKDV_ARGS);
  else dkdv_kernel<T, D, 64><<<a.BH * m->Tk, 256, 0, a.s>>>(SA2_DKDV_ARGS);
#undef SA2_DKDV_ARGS
}

template <typename T, int D> struct DqLaunch { static void run(const BwdArgs& a) { launch_dq<T, D>(a); } };
template <typename T, int D> struct DkdvLaunch { static void run(const BwdArgs& a) { launch_dkdv<T, D>(a); } };

template <template <typename, int> class F>
static void by_type(int dtype, int d, const BwdArgs& a) {
  if (dtype == SA2_BF16) {
    if (d == 128) F<bf16_t, 128>::run(a); else F<bf16_t, 64>::run(a);
  } else {
    if (d == 128) F<float, 128>::run(a); else F<float, 64>::run(a);
  }
}

// Workspace regions of the backward, each 256-byte aligned: the row
// statistics; for d = 128 also the partial slots of split dQ rows and of
// split dK/dV columns.
struct BwdWorkspace {
  size_t stats, dq_partials, dkdv_partials, total;
};
static BwdWorkspace bwd_workspace(int B, int H, int N, int d) {
  BwdWorkspace w{};
  w.stats = 0;
  size_t off = up256((size_t)B * H * stat_groups(N) * 256);
  if (d == 128) {
    w.dq_partials = off;
    off = up256(off + partial_bytes(kRowPlan, kDqPartialFloats));
    w.dkdv_partials = off;
    off = up256(off + partial_bytes(kColPlan, kPartialFloats));
  }
  w.total = off;
  return w;
}

static sa2_status check_bwd(const char* fn, const void* q, const void* k, const void* v,
                            const float* lse, const void* dout, int dtype, int B, int H, int N,
                            int d, const sa2_mask* m, void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !lse || !dout || !ws) return fail(SA2_EINVAL, std::string(fn) + ": null pointer");
  if (sa2_status st = check_common(fn, dtype, B, H, N, d, m)) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(dout))
    return fail(SA2_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(SA2_EINVAL, std::string(fn) + ": workspace not 256-byte aligned");
  if (ws_bytes < sa2_bwd_workspace_bytes(B, H, N, d))
    return fail(SA2_EINVAL, std::string(fn) + ": workspace smaller than sa2_bwd_workspace_bytes()");
  return SA2_OK;
}


static BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, int B, int H, int N, int d,
                        const sa2_mask* m, void* dq, void* dk, void* dv, void* ws, void* stream) {
  const double sc = 1.0 / sqrt((double)d);
  const BwdWorkspace w = bwd_workspace(B, H, N, d);
  char* base = static_cast<char*>(ws);
  BwdArgs a{q, k, v, o, dout, lse, m, B * H, N, (float)(1.4426950408889634 * sc), (float)sc,
            dq, dk, dv, reinterpret_cast<float*>(base + w.stats), PlanPtrs{}, PlanPtrs{},
            reinterpret_cast<hipStream_t>(stream)};
  if (d == 128) {
    a.rows = plan_ptrs(m->row_plan, B * H * m->Tq, kRowPlan, kRowCounters, 1,
                       reinterpret_cast<float*>(base + w.dq_partials));
    a.cols = plan_ptrs(m->col_plan, B * H * m->Tk, kColPlan, kColCounters, 0,
                       reinterpret_cast<float*>(base + w.dkdv_partials));
  }
  return a;
}

}  // namespace sa2

using namespace sa2;

extern "C" size_t sa2_fwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return d == 128 ? up256(partial_bytes(kRowPlan, kFwdPartialFloats)) : 0;
}

extern "C" sa2_status sa2_attn_fwd(const void* q, const void* k, const void* v, int dtype, int B,
                                   int H, int N, int d, const sa2_mask* m, void* o, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return fail(SA2_EINVAL, "sa2_attn_fwd: null pointer");
  if (sa2_status st = check_common("sa2_attn_fwd", dtype, B, H, N, d, m)) return st;
  if (!m->row_cnt || !m->row_idx) return fail(SA2_EINVAL, "sa2_attn_fwd: mask row lists are null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(SA2_EINVAL, "sa2_attn_fwd: pointers must be 16-byte aligned");
  const size_t need = sa2_fwd_workspace_bytes(B, H, N, d);
  if (need > 0) {
    if (!ws) return fail(SA2_EINVAL, "sa2_attn_fwd: null workspace");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
      return fail(SA2_EINVAL, "sa2_attn_fwd: workspace not 256-byte aligned");
    if (ws_bytes < need)
      return fail(SA2_EINVAL, "sa2_attn_fwd: workspace smaller than sa2_fwd_workspace_bytes()");
  }
  const bool planned = dtype == SA2_BF16 && d == 128;
  if (planned && (!m->row_plan || !aligned16(m->row_plan)))
    return fail(SA2_EINVAL, "sa2_attn_fwd: mask row plan is null or misaligned (bf16, d = 128)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int BH = B * H;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)d));
  const PlanPtrs rp = planned ? plan_ptrs(m->row_plan, BH * m->Tq, kRowPlan, kRowCounters, 0,
                                          static_cast<float*>(ws))
                              : PlanPtrs{};
  if (dtype == SA2_BF16) {
    if (d == 128) dispatch_fwd<bf16_t, 128>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
    else dispatch_fwd<bf16_t, 64>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
  } else {
    if (d == 128) dispatch_fwd<float, 128>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
    else dispatch_fwd<float, 64>(q, k, v, m, BH, N, sl2, o, lse, rp, s);
  }
  return check_launch("fwd_kernel");
}


extern "C" size_t sa2_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return sa2::bwd_workspace(B, H, N, d).total;
}

extern "C" sa2_status sa2_attn_bwd_dq(const void* q, const void* k, const void* v,
                                      const void* o, const float* lse, const void* dout,
                                      int dtype, int B, int H, int N, int d, const sa2_mask* m,
                                      void* dq, void* ws, size_t ws_bytes, void* stream) {
  if (sa2_status st = check_bwd("sa2_attn_bwd_dq", q, k, v, lse, dout, dtype, B, H, N, d, m, ws,
                                ws_bytes))
    return st;
  if (!o || !dq) return fail(SA2_EINVAL, "sa2_attn_bwd_dq: null pointer");
  if (!aligned16(o) || !aligned16(dq))
    return fail(SA2_EINVAL, "sa2_attn_bwd_dq: pointers must be 16-byte aligned");
  if (!m->row_cnt || !m->row_idx) return fail(SA2_EINVAL, "sa2_attn_bwd_dq: mask row lists are null");
  if (dtype == SA2_BF16 && d == 128 && (!m->row_plan || !aligned16(m->row_plan)))
    return fail(SA2_EINVAL, "sa2_attn_bwd_dq: mask row plan is null or misaligned (bf16, d = 128)");
  by_type<DqLaunch>(dtype, d, bwd_args(q, k, v, o, lse, dout, B, H, N, d, m, dq, nullptr, nullptr, ws, stream));
  return check_launch("dq_kernel");
}

extern "C" sa2_status sa2_attn_bwd_dkdv(const void* q, const void* k, const void* v,
                                        const float* lse, const void* dout, int dtype, int B,
                                        int H, int N, int d, const sa2_mask* m, void* dk,
                                        void* dv, void* ws, size_t ws_bytes, void* stream) {
  if (sa2_status st = check_bwd("sa2_attn_bwd_dkdv", q, k, v, lse, dout, dtype, B, H, N, d, m,
                                ws, ws_bytes))
    return st;
  if (!dk || !dv) return fail(SA2_EINVAL, "sa2_attn_bwd_dkdv: null pointer");
  if (!aligned16(dk) || !aligned16(dv))
    return fail(SA2_EINVAL, "sa2_attn_bwd_dkdv: pointers must be 16-byte aligned");
  if (!m->col_cnt || !m->col_idx) return fail(SA2_EINVAL, "sa2_attn_bwd_dkdv: mask column lists are null");
  if (dtype == SA2_BF16 && d == 128 && (!m->col_plan || !aligned16(m->col_plan)))
    return fail(SA2_EINVAL,
                "sa2_attn_bwd_dkdv: mask column plan is null or misaligned (bf16, d = 128)");
  by_type<DkdvLaunch>(dtype, d, bwd_args(q, k, v, nullptr, lse, dout, B, H, N, d, m, nullptr, dk, dv, ws, stream));
  return check_launch("dkdv_kernel");
}

extern "C" size_t sa2_bwd_atomic_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d != 128) return 0;
  return sa2::bwd_workspace(B, H, N, d).total + up256((size_t)B * H * N * d * sizeof(float));
}

extern "C" sa2_status sa2_attn_bwd_atomic_dq(const void* q, const void* k, const void* v,
                                             const void* o, const float* lse, const void* dout,
                                             int dtype, int B, int H, int N, int d,
                                             const sa2_mask* m, void* dq, void* dk, void* dv,
                                             void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sa2_attn_bwd_atomic_dq";
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !ws)
    return fail(SA2_EINVAL, std::string(fn) + ": null pointer");
  if (sa2_status st = check_common(fn, dtype, B, H, N, d, m)) return st;
  if (dtype != SA2_BF16 || d != 128)
    return fail(SA2_EUNSUPPORTED, std::string(fn) + ": bf16 with d = 128 only");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(SA2_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(SA2_EINVAL, std::string(fn) + ": workspace not 256-byte aligned");
  if (ws_bytes < sa2_bwd_atomic_workspace_bytes(B, H, N, d))
    return fail(SA2_EINVAL,
                std::string(fn) + ": workspace smaller than sa2_bwd_atomic_workspace_bytes()");
  if (!m->col_cnt || !m->col_idx || !m->col_plan || !aligned16(m->col_plan))
    return fail(SA2_EINVAL, std::string(fn) + ": mask column lists or plan missing");
  const BwdArgs a = bwd_args(q, k, v, o, lse, dout, B, H, N, d, m, dq, dk, dv, ws, stream);
  float* dq_acc =
      reinterpret_cast<float*>(static_cast<char*>(ws) + bwd_workspace(B, H, N, d).total);
  const int G4 = stat_groups(N) / 4;
  dq_prep_kernel<<<a.BH * G4, 256, 0, a.s>>>(static_cast<const bf16_t*>(o),
                                             static_cast<const bf16_t*>(dout), lse, a.stats,
                                             dq_acc, N, G4);
  const int ncols = a.BH * m->Tk;
  const int grid = 8 * plan_items_per_xcd(ncols, kColPlan);
#define SA2_DKDV_FUSED_ARGS                                                                  \
  static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), \
      static_cast<const bf16_t*>(dout), a.stats, a.cols.items, m->col_idx, N, m->Tq, m->Tk,    \
      a.sl2, a.scale, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), a.cols.splits,       \
      a.cols.done, a.cols.partials, ncols, dq_acc
  if (m->bq == 128) dkdv_pair_kernel<128, true><<<grid, 128, 0, a.s>>>(SA2_DKDV_FUSED_ARGS);
  else dkdv_pair_kernel<64, true><<<grid, 128, 0, a.s>>>(SA2_DKDV_FUSED_ARGS);
#undef SA2_DKDV_FUSED_ARGS
  const size_t n4 = (size_t)a.BH * N * d / 4;
  dq_finish_kernel<<<(unsigned)std::min<size_t>((n4 + 255) / 256, 8192), 256, 0, a.s>>>(
      dq_acc, n4, a.scale, static_cast<bf16_t*>(dq));
  return check_launch("dkdv_pair_kernel (fused dQ)");
}

extern "C" sa2_status sa2_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, int dtype, int B, int H,
                                   int N, int d, const sa2_mask* m, void* dq, void* dk, void* dv,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (sa2_status st = sa2_attn_bwd_dq(q, k, v, o, lse, dout, dtype, B, H, N, d, m, dq, ws,
                                      ws_bytes, stream))
    return st == SA2_OK ? st : fail(st, std::string("sa2_attn_bwd: ") + sa2_last_error());
  if (sa2_status st = sa2_attn_bwd_dkdv(q, k, v, lse, dout, dtype, B, H, N, d, m, dk, dv, ws,
                                        ws_bytes, stream))
    return fail(st, std::string("sa2_attn_bwd: ") + sa2_last_error());
  return SA2_OK;
}
