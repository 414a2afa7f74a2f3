// Work plans of the attention kernels (gfx950 / CDNA4).  Shared by the mask
// builder, which writes a mask's plans once, and the attention kernels,
// which walk them.
#pragma once

#include "sa2_common.h"

namespace sa2 {

// A list length read from a mask, clamped to [0, cap]: a malformed mask
// then gives wrong values but no access past the lists and no unbounded loop.
__device__ inline int list_len(int n, int cap) { return min(max(n, 0), cap); }

// ---------------------------------------------------------------------------
// Work plans.  One workgroup walks one list (a query block's row list in the
// forward and dQ kernels, a key block's column list in the dK/dV kernel), so
// a long list would set a kernel's time by itself: an attention sink is kept
// by every query block, and under Top-p a few rows of a skewed head keep most
// key blocks (gist.science section 1).  A plan cuts every list longer than L
// into nearly equal segments; a segment's workgroup writes fp32 partial sums
// to a slot of the workspace and counts itself done on the list's completion
// counter; the workgroup that finds itself last combines the list's partials
// in segment order and writes the outputs.  Values are never accumulated
// atomically and the order of every sum is fixed, so results are
// reproducible bit for bit; no workgroup waits for another.
//
// L is the larger of `min_segment` and `fair` times the mean load of the
// kernel's resident workgroups (`slots`), so that only lists that would set
// the kernel's time are cut (each cut costs a partial write, a device-scope
// release and the final combine), and per XCD share at least total / `extra`,
// which bounds a share's extra segments by `extra` and its partial slots by
// 2 `extra`.
//
// Items, in the mask's plan array as int4 {list, first list entry, entries, -1 or
// split entry * 1024 + segment}; item j of XCD x sits at 8j + x (the
// workgroup slots that run on XCD x), longest first; unused items have list
// -1.  Each XCD takes a contiguous share of the lists, so its L2 sees a
// narrow band of heads.  Shares are cut at equal cost (list length + 1)
// rather than equal count where the equal-count shares are unbalanced:
// densities differ from head to head, and under a skewed mask the long lists
// of one head would otherwise all fall to one XCD, whose share would set the
// kernel's time.  Split entries: int4 {list, first partial slot, segments},
// `extra` per XCD share.
// ---------------------------------------------------------------------------
struct PlanKind {
  int slots;        // resident workgroups of the kernel that walks the lists
  int fair;         // lists up to this many mean loads stay whole
  int extra;        // extra segments (and split lists) per XCD share
  int min_segment;  // shortest segment worth its own workgroup
  int imbalance;    // XCD shares are cut at equal cost when the costliest
                    // equal-count share exceeds the mean by more than this
                    // many percent (0: always), else at equal count
  int quarters;     // head-major groups give XCD 4g + r the r-th quarter of
                    // every head's lists (1), or deal their items in turn (0)
};
// dK/dV: 256 CUs x 4 workgroups.  Forward and dQ: 256 CUs x 2; a row
// segment also pays a combine pass over every segment of its row, so rows
// are cut no finer than 16 key blocks.  Equal-count row shares keep whole
// heads together in an XCD's L2 (the cost-balanced cut measured 4% slower
// on a mask whose heads differ by a few percent), so rows are balanced only
// when a share would carry over 10% more than its part.
constexpr PlanKind kColPlan{1024, 2, 128, 8, 0, 0};
constexpr PlanKind kRowPlan{512, 1, 64, 16, 10, 1};
constexpr int kPlanBuckets = 4096;   // list lengths are ranked by min(length, 4095)
constexpr size_t kPartialFloats = 2 * 64 * 128;           // dV and dK of one key block
constexpr size_t kFwdPartialFloats = 128 * 128 + 2 * 128;  // O of a query block, m, l
constexpr size_t kDqPartialFloats = 128 * 128;             // dQ of a query block

// Cost-balanced shares move a boundary at most share_slack(n) items from the
// equal-count one.
__host__ __device__ inline int share_slack(int n) { return ((n + 7) / 8 + 15) / 16; }
__host__ __device__ inline int plan_items_per_xcd(int n, PlanKind k) {
  return (n + 7) / 8 + 2 * share_slack(n) + k.extra;
}

// Inclusive scan of v over the workgroup (threads in order): a shuffle scan
// in each wave, then the wave totals through LDS (tot: one entry per wave).
// Returns the thread's inclusive sum and sets *all to the workgroup's total.
template <typename T>
__device__ inline T block_scan(T v, T* tot, T* all) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) tot[w] = v;
  __syncthreads();
  T before = 0, sum = 0;
  for (int i = 0; i < nw; ++i) {
    const T t = tot[i];
    before += i < w ? t : 0;
    sum += t;
  }
  __syncthreads();   // tot may be reused
  *all = sum;
  return v + before;
}

// The plan of XCD share x of n lists (lengths cnt, each at most cap;
// `per_head` consecutive lists belong to one (batch, head)), by one workgroup
// of nt threads (a multiple of 64 that divides kPlanBuckets).  LDS:
// hist[kPlanBuckets] ints, itot and red (nt / 64 entries each), ctr[6],
// pos[20] 64-bit.
//
// Shares.  One pass gives every thread the cost (list length + 1) of a
// contiguous chunk of the lists; a scan of the chunks gives the total and,
// at the equal-count boundaries E(k) = k n / 8 (rounded as the lists are
// dealt), the eight equal-count share costs.  Cost-balanced boundaries are
// the first list whose predecessors cost at least k / 8 of the total,
// clamped to within share_slack(n) lists of E(k).  XCDs 4g .. 4g+3 form
// group g, whose share is the union of theirs.
//
// Order.  A group is planned head by head when no item of its share is
// longer than a quarter of the group's mean load per resident workgroup
// (share cost over slots / 2): the group's items go one (batch, head) after
// another, longest first within each, so that the four XCDs work on one head
// at a time and its tiles are shared through the last-level cache while they
// are live (14B-shaped layer: forward -14%, dQ -8%, dK/dV -19% against
// per-XCD longest-first order).  In the row plan XCD 4g + r takes the r-th
// contiguous quarter of every head's lists, so that an XCD's query blocks of
// a head are neighbours, which keep more K/V tiles in common (forward -1.3%
// and -2.5%, dQ -1.7% and -1.2% at the 1.3B and 14B layers against dealing
// the items to the four XCDs in turn); the column plan deals its items in
// turn (quarters made dK/dV 8% slower at the 14B layer).  When a quarter
// would hold more items than an XCD has slots (few lists per head, not a
// multiple of four), the items are dealt in turn as well.  The group's
// first workgroup writes the whole group.  Where some item is longer, a list
// that starts late would set the kernel's time (the 1.3B layer's longest
// columns are as long as a slot's whole load), so each XCD takes its own
// share longest first.  Quarters, heads and lengths share the kPlanBuckets
// ranks: with nh heads in the share, each (quarter, head) has
// kPlanBuckets / (4 nh) length ranks (kPlanBuckets / nh when dealt in turn),
// exact when that exceeds the longest item.
static __device__ void plan_share(int x, const int32_t* __restrict__ cnt, int n, int cap,
                                  int per_head, PlanKind kd, int4* __restrict__ items,
                                  int4* __restrict__ splits, int* __restrict__ done, int ndone,
                                  int* hist, int* itot, long long* red, int* ctr,
                                  long long* pos) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  auto cost = [&](int i) { return (long long)list_len(cnt[i], cap) + 1; };
  long long csum = 0;
#pragma unroll 4
  for (int i = lo; i < hi; ++i) csum += cost(i);
  if (tid < 20) pos[tid] = 0;
  long long total;
  const long long run = block_scan(csum, red, &total) - csum;
  const int q8 = n / 8, r8 = n % 8;
  auto eq = [&](int k) { return k * q8 + min(k, r8); };
  // pos[k] (k = 0..8): prefix cost at E(k), by the thread whose chunk holds it
  for (int k = 0; k <= 8; ++k) {
    const int e = eq(k);
    if ((e < n && e >= lo && e < hi) || (e == n && tid == nt - 1)) {
      long long acc = run;
      for (int i = lo; i < min(e, hi); ++i) acc += cost(i);
      pos[k] = e == n ? total : acc;
    }
  }
  __syncthreads();
  long long worst = 0;
  for (int k = 0; k < 8; ++k) worst = max(worst, pos[k + 1] - pos[k]);
  const bool balanced = kd.imbalance == 0 || worst * 800 > total * (800 + 8 * kd.imbalance);
  // boundaries: 0, 1 of XCD share x; 2, 3 of its group
  const int grp = x >> 2;
  auto bidx = [&](int k) { return k == 0 ? x : k == 1 ? x + 1 : k == 2 ? 4 * grp : 4 * grp + 4; };
  int b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = eq(bidx(k));
  if (balanced) {
    // pos[10 + k]: first list whose predecessors cost at least bidx(k) / 8 of the total
    if (tid < 4) pos[10 + tid] = bidx(tid) == 0 ? 0 : n;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long long target = ((long long)bidx(k) * total + 7) / 8;
      if (target > 0 && run < target && target <= run + csum) {
        long long acc = run;
        int bb = hi;
        for (int i = lo; i < hi; ++i) {
          if (acc >= target) { bb = i; break; }
          acc += cost(i);
        }
        pos[10 + k] = bb;
      }
    }
    __syncthreads();
    const int H = share_slack(n);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      b[k] = min(max((int)pos[10 + k], max(0, b[k] - H)), min(n, b[k] + H));
  }

  // list entries and the longest list, over XCD share x and over the group
  long long mine = 0, gmine = 0;
  int glong = 0;
  for (int i = b[0] + tid; i < b[1]; i += nt) mine += list_len(cnt[i], cap);
  for (int i = b[2] + tid; i < b[3]; i += nt) {
    const int ln = list_len(cnt[i], cap);
    gmine += ln;
    glong = max(glong, ln);
  }
  for (int off = 32; off > 0; off >>= 1) {
    mine += __shfl_xor(mine, off);
    gmine += __shfl_xor(gmine, off);
    glong = max(glong, __shfl_xor(glong, off));
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    red[tid >> 6] = mine;
    itot[tid >> 6] = glong;
  }
  __syncthreads();
  long long share = 0;
  int glongest = 0;
  for (int w = 0; w < nt / 64; ++w) {
    share += red[w];
    glongest = max(glongest, itot[w]);
  }
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = gmine;
  __syncthreads();
  long long gshare = 0;
  for (int w = 0; w < nt / 64; ++w) gshare += red[w];
  __syncthreads();   // red and itot are reused below

  const long long all = total - n;
  const long long Lg =
      max((long long)kd.min_segment, kd.fair * ((all + kd.slots - 1) / kd.slots));
  auto nseg_at = [](int ln, int L) { return ln > L ? (ln + L - 1) / L : 1; };
  const int Lgrp = (int)max(Lg, (gshare + 4 * kd.extra - 1) / (4 * kd.extra));
  const int gseg = (glongest + nseg_at(glongest, Lgrp) - 1) / nseg_at(glongest, Lgrp);
  const int G0 = b[2], G1 = b[3];
  const bool head_major =
      G1 > G0 && 4LL * gseg * (kd.slots / 2) <= gshare + (long long)(G1 - G0);
  if (head_major && (x & 3) != 0) return;   // the group's first workgroup plans it

  // the lists to place, their cut, and where split entries and partial slots come from
  const int c0 = head_major ? G0 : b[0], len = head_major ? G1 - G0 : b[1] - b[0];
  const int L = head_major ? Lgrp : (int)max(Lg, (share + kd.extra - 1) / kd.extra);
  const int ebase = head_major ? 4 * kd.extra * grp : kd.extra * x;
  const int pbase = 2 * ebase;
  const int ecap = head_major ? 4 * kd.extra : kd.extra;
  auto nseg = [&](int ln) { return nseg_at(ln, L); };
  auto seg = [&](int ln, int ns, int s, int& start) {
    const int base = ln / ns, rem = ln % ns;
    start = s * base + min(s, rem);
    return base + (s < rem ? 1 : 0);
  };
  const int ph = max(per_head, 1);
  // quarter of list id within its (batch, head): (index in head) * 4 / ph,
  // by comparisons rather than a division
  auto quarter = [&](int id) {
    const int j4 = 4 * (id - (id / ph) * ph);
    return (j4 >= ph ? 1 : 0) + (j4 >= 2 * ph ? 1 : 0) + (j4 >= 3 * ph ? 1 : 0);
  };
  const int J = plan_items_per_xcd(n, kd);
  // rank bucket of an item (higher buckets are placed first): its length, or
  // for a head-major group (quarter, head, length), or (head, length) when
  // dealt in turn
  const int h0 = c0 / ph;
  const int nh = len > 0 ? (c0 + len - 1) / ph - h0 + 1 : 1;
  bool quarters = head_major && kd.quarters;   // until a quarter overflows
  int nr = quarters ? 4 * nh : nh;             // (quarter,) head ranks
  int nb = nr <= kPlanBuckets ? kPlanBuckets / nr : 1;
  auto bucket = [&](int id, int sl) {
    if (!head_major) return min(sl, kPlanBuckets - 1);
    const int hh = (quarters ? quarter(id) * nh : 0) + id / ph - h0;
    const int hb = nr <= kPlanBuckets ? hh : (int)((long long)hh * kPlanBuckets / nr);
    const int lr = nb - 1 - min(nb - 1, (int)((long long)sl * nb / (gseg + 1)));
    return kPlanBuckets - 1 - (hb * nb + lr);
  };
  // histogram of the items' buckets, with the items per quarter (ctr[2 + r])
  auto histogram = [&](bool count_quarters) {
    for (int c = tid; c < kPlanBuckets; c += nt) hist[c] = 0;
    if (tid < 6) ctr[tid] = 0;
    __syncthreads();
    int qn[4] = {0, 0, 0, 0};
    for (int j = tid; j < len; j += nt) {
      const int id = c0 + j, ln = list_len(cnt[id], cap), ns = nseg(ln);
      for (int s2 = 0; s2 < ns; ++s2) {
        int st;
        atomicAdd(&hist[bucket(id, seg(ln, ns, s2, st))], 1);
      }
      const int r = quarter(id);
#pragma unroll
      for (int i = 0; i < 4; ++i) qn[i] += r == i ? ns : 0;
    }
    if (count_quarters) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        for (int off = 32; off > 0; off >>= 1) qn[i] += __shfl_xor(qn[i], off);
        if ((tid & 63) == 0) atomicAdd(&ctr[2 + i], qn[i]);
      }
    }
    __syncthreads();
  };
  histogram(quarters);
  if (quarters && max(max(ctr[2], ctr[3]), max(ctr[4], ctr[5])) > J) {
    quarters = false;   // a quarter would overflow its XCD's item slots: deal in turn
    nr = nh;
    nb = nr <= kPlanBuckets ? kPlanBuckets / nr : 1;
    __syncthreads();
    histogram(false);
  }
  int qstart[4];
  qstart[0] = 0;
#pragma unroll
  for (int r = 1; r < 4; ++r) qstart[r] = qstart[r - 1] + ctr[1 + r];
  // item k of the order (k counts from the first item of the item's
  // quarter): slot 8k + x, or 8k + 4g + r in quarter r, or dealt in turn
  auto slot_of = [&](int k, int id) {
    if (!head_major) return 8 * k + x;
    if (quarters) {
      const int r = quarter(id);
      return 8 * (k - qstart[r]) + 4 * grp + r;
    }
    return 8 * (k >> 2) + 4 * grp + (k & 3);
  };
  // the first position of each bucket in descending bucket order
  const int bper = kPlanBuckets / nt;   // nt divides kPlanBuckets
  const int blo = tid * bper, bhi = blo + bper;
  int local = 0;
  for (int r = blo; r < bhi; ++r) local += hist[kPlanBuckets - 1 - r];
  int nitems;
  int brun = block_scan(local, itot, &nitems) - local;
  for (int r = blo; r < bhi; ++r) {
    const int c = kPlanBuckets - 1 - r;
    const int h = hist[c];
    hist[c] = brun;
    brun += h;
  }
  __syncthreads();
  for (int j = tid; j < len; j += nt) {
    const int id = c0 + j, ln = list_len(cnt[id], cap), ns = nseg(ln);
    int entry = -1;
    if (ns > 1) {
      const int p0 = pbase + atomicAdd(&ctr[1], ns);
      entry = ebase + atomicAdd(&ctr[0], 1);
      splits[entry] = make_int4(id, p0, ns, 0);
    }
    for (int s2 = 0; s2 < ns; ++s2) {
      int st;
      const int sl = seg(ln, ns, s2, st);
      items[slot_of(atomicAdd(&hist[bucket(id, sl)], 1), id)] =
          make_int4(id, st, sl, ns > 1 ? entry * 1024 + s2 : -1);
    }
  }
  __syncthreads();
  // unused items of the XCDs planned here, unused split entries, counters
  for (int r = 0; r < (head_major ? 4 : 1); ++r) {
    const int used = quarters ? ctr[2 + r]
                     : head_major ? (nitems > r ? (nitems - r + 3) / 4 : 0) : nitems;
    const int col = head_major ? 4 * grp + r : x;
    for (int j = used + tid; j < J; j += nt) items[8 * j + col] = make_int4(-1, 0, 0, -1);
  }
  for (int j = ctr[0] + tid; j < ecap; j += nt) splits[ebase + j] = make_int4(-1, 0, 0, 0);
  for (int a = 0; a < ndone; ++a)
    for (int j = tid; j < ecap; j += nt) done[8 * kd.extra * a + ebase + j] = 0;
}

// A plan item checked against the call: {list, first entry, entries, split}
// with the split entry it names (sp = {list, first partial slot, segments}).
// An item that does not fit (a plan written for another mask, or never
// written) is refused, so nothing is read or written out of range.
__device__ inline bool plan_item_ok(const int4 item, int nlists, int cap, PlanKind kd,
                                    const int4* __restrict__ splits, int4& sp) {
  if (item.x < 0 || item.x >= nlists || item.y < 0 || item.z < 0 || item.y + item.z > cap)
    return false;
  sp = make_int4(0, 0, 0, 0);
  if (item.w < 0) return true;
  const int entry = item.w >> 10, seg = item.w & 1023;
  if (entry >= 8 * kd.extra) return false;
  sp = splits[entry];
  return sp.x == item.x && sp.y >= 0 && sp.z >= 2 && seg < sp.z && sp.y + sp.z <= 16 * kd.extra;
}


// Byte offsets of a plan in its int32 array: items, split entries, then
// `ndone` counter arrays.
struct PlanLayout {
  size_t items, splits, done, bytes;
};
__host__ __device__ inline PlanLayout plan_layout(int n, PlanKind kd, int ndone) {
  PlanLayout l;
  l.items = 0;
  l.splits = (size_t)8 * plan_items_per_xcd(n, kd) * sizeof(int4);
  l.done = l.splits + (size_t)8 * kd.extra * sizeof(int4);
  l.bytes = l.done + (size_t)ndone * 8 * kd.extra * sizeof(int);
  return l;
}
constexpr int kRowCounters = 2;   // forward, dQ
constexpr int kColCounters = 1;   // dK/dV

}  // namespace sa2
