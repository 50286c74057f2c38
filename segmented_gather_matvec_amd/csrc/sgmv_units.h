// sgmv_units.h - mapping of a workgroup's unit number to its rows and LoRA.
//
// A unit is one block of at most RB consecutive rows of one segment.  Units
// are numbered segment by segment.  When every segment fits one block the
// unit number is the segment number ("direct"); otherwise each wave scans the
// segment lengths (64 segments at a time) to find the segment that holds the
// unit.  Metadata that breaks the documented preconditions yields an empty
// unit instead of an out-of-range access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgmv {

struct Unit {
  int r0;  // first row
  int L;   // rows (0: nothing to do)
  int k;   // LoRA id
};

// Map unit u to its segment, first row and row count.  With direct units the
// unit is the segment; otherwise every wave scans ceil(len_s / RB) over the
// segments (64 at a time) and finds the segment whose unit range holds u.
template <int RB>
__device__ inline Unit resolve_unit(const int32_t* seg_indptr, const int32_t* lora_idx, int num_segs,
                                   int num_loras, int n_rows, int direct_units, int u) {
  Unit out{0, 0, 0};
  int s = -1, rb = 0;
  if (direct_units) {
    if (u < num_segs) s = u;
  } else {
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int c0 = 0; c0 < num_segs; c0 += 64) {
      const int sl = c0 + lane;
      int units = 0;
      if (sl < num_segs) {
        int len = seg_indptr[sl + 1] - seg_indptr[sl];
        len = len > 0 ? len : 0;
        units = (len + RB - 1) / RB;
      }
      int incl = units;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
      }
      const int excl = incl - units;
      const bool hit = sl < num_segs && u >= base + excl && u < base + incl;
      const unsigned long long m = __ballot(hit);
      if (m) {
        const int l = __builtin_ctzll(m);
        s = c0 + l;
        rb = u - base - __shfl(excl, l, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  rb = __builtin_amdgcn_readfirstlane(rb);
  if (s < 0) return out;
  const int lo = seg_indptr[s];
  const int hi = seg_indptr[s + 1];
  const int k = lora_idx[s];
  const int r0 = lo + rb * RB;
  int r1 = hi < r0 + RB ? hi : r0 + RB;
  r1 = r1 < n_rows ? r1 : n_rows;
  // One combined test (no short circuit), so that the three loads above are
  // issued together rather than split around an early exit on r0.
  const bool bad = (r0 < 0) | (r1 <= r0) | (k < 0) | (k >= num_loras);
  if (bad) return out;
  out.r0 = r0;
  out.L = r1 - r0;
  out.k = k;
  return out;
}

// resolve_unit for at most 64 segments whose bounds are already in registers:
// lane l holds lo_l = seg_indptr[l] and hi_l = seg_indptr[l + 1] (lanes at or
// past num_segs hold anything).  The returned k is the unit's segment.
template <int RB>
__device__ inline Unit resolve_unit_lanes(int lo_l, int hi_l, int num_segs, int n_rows, int direct_units,
                                          int u) {
  Unit out{0, 0, 0};
  const int lane = threadIdx.x & 63;
  int s = -1, rb = 0;
  if (direct_units) {
    if (u < num_segs) s = u;
  } else {
    int units = 0;
    if (lane < num_segs) {
      const int len = hi_l - lo_l > 0 ? hi_l - lo_l : 0;
      units = (len + RB - 1) / RB;
    }
    int incl = units;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      if (lane >= d) incl += up;
    }
    const int excl = incl - units;
    const bool hit = lane < num_segs && u >= excl && u < incl;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int l = __builtin_ctzll(m);
      s = l;
      rb = u - __shfl(excl, l, 64);
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  rb = __builtin_amdgcn_readfirstlane(rb);
  if (s < 0 || s >= 64) return out;
  const int lo = __builtin_amdgcn_readlane(lo_l, s);
  const int hi = __builtin_amdgcn_readlane(hi_l, s);
  const int r0 = lo + rb * RB;
  int r1 = hi < r0 + RB ? hi : r0 + RB;
  r1 = r1 < n_rows ? r1 : n_rows;
  if ((r0 < 0) | (r1 <= r0)) return out;
  out.r0 = r0;
  out.L = r1 - r0;
  out.k = s;
  return out;
}

// Rank of a LoRA as used by the kernels: the stored value clamped to [0, R]
// and rounded down to a multiple of 8 (one 128-bit vector of A_k per 8 ranks).
template <int R>
__device__ inline int lora_rank(int r) {
  return (r < 0 ? 0 : r > R ? R : r) & ~7;
}


}  // namespace sgmv
