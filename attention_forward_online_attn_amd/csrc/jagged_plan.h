// On-device tile plan for the jagged layout: the compact list of
// (sequence, query tile) work items, ordered by the number of key tiles each
// must visit, largest first.
//
// The SLL jagged page launches one program per (query tile up to
// max_seq_len, batch x head) and lets programs past a sequence's length exit
// (_multi_head_jagged_flash_attention_fwd_kernel's early return).  With
// lengths spread over 1..max_seq_len most of those programs are empty and the
// long sequences' tiles can start last.  Here one small workgroup reads the
// offsets on the device (no host sync), counting-sorts the non-empty items by
// cost and writes the list; the forward kernel's grid covers an upper bound
// of the item count and maps workgroup i to item i / H, head i % H, so the
// heaviest tiles are dispatched first, and a sequence's tiles of equal cost
// are dispatched back to back.
#pragma once

#include "attn_common.h"

namespace attn {

constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 1024;  // cost buckets; costs above share the last bucket

// Key tiles a (sequence, query tile) item visits; 0 when none of its rows
// attends (rows past max_seq_len).
__device__ __forceinline__ int item_cost(int qt, int used, int causal, int BM, int BN) {
  const int r0 = qt * BM;
  if (r0 >= used) return 0;
  const int lim = causal ? min(r0 + BM, used) : used;
  return (lim + BN - 1) / BN;
}

// plan layout (int32): [0] = item count, [1..3] unused, then (seq, q-tile)
// pairs.  `capacity` is the number of pairs the buffer holds.
__global__ void __launch_bounds__(kPlanThreads)
jagged_plan_kernel(const int64_t* offsets, int num_seqs, int64_t total_len, int max_seq_len,
                   int causal, int BM, int BN, int32_t* plan, int capacity) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int scan[kPlanBuckets];
  const int tid = threadIdx.x;
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();

  // pass 1: histogram of item costs
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    int64_t b = offsets[s], e = offsets[s + 1];
    b = b < 0 ? 0 : (b > total_len ? total_len : b);
    e = e < b ? b : (e > total_len ? total_len : e);
    const int len = (int)(e - b);
    const int used = len < max_seq_len ? len : max_seq_len;
    const int nq = (len + BM - 1) / BM;
    for (int qt = 0; qt < nq; ++qt) {
      const int c = min(item_cost(qt, used, causal, BM, BN), kPlanBuckets - 1);
      atomicAdd(&hist[c], 1);
    }
  }
  __syncthreads();

  // exclusive scan over buckets in DESCENDING cost order: bucket c starts
  // after all buckets with larger cost.  Slot i holds bucket (NB - 1 - i).
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) scan[i] = hist[kPlanBuckets - 1 - i];
  __syncthreads();
  for (int step = 1; step < kPlanBuckets; step <<= 1) {  // inclusive Hillis-Steele scan
    int add = 0;
    if (tid < kPlanBuckets && tid >= step) add = scan[tid - step];
    __syncthreads();
    if (tid < kPlanBuckets) scan[tid] += add;
    __syncthreads();
  }
  // start of bucket c = inclusive prefix up to slot (NB - 1 - c), minus its own count
  for (int c = tid; c < kPlanBuckets; c += kPlanThreads) hist[c] = scan[kPlanBuckets - 1 - c] - hist[c];
  if (tid == 0) {
    const int total = scan[kPlanBuckets - 1];
    plan[0] = total < capacity ? total : capacity;
  }
  __syncthreads();

  // pass 2: scatter the items to their bucket's range.  A sequence's
  // consecutive tiles of equal cost (all its tiles without causal masking)
  // take one contiguous run of positions, so they are dispatched back to
  // back: with H a multiple of 8, workgroup (item H + h) of every tile of a
  // (sequence, head) lands on the same XCD, and those tiles read the
  // sequence's K/V through one L2 instead of each fetching it from HBM.
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    int64_t b = offsets[s], e = offsets[s + 1];
    b = b < 0 ? 0 : (b > total_len ? total_len : b);
    e = e < b ? b : (e > total_len ? total_len : e);
    const int len = (int)(e - b);
    const int used = len < max_seq_len ? len : max_seq_len;
    const int nq = (len + BM - 1) / BM;
    for (int qt = 0; qt < nq;) {
      const int c = min(item_cost(qt, used, causal, BM, BN), kPlanBuckets - 1);
      int run = 1;
      while (qt + run < nq && min(item_cost(qt + run, used, causal, BM, BN), kPlanBuckets - 1) == c) ++run;
      const int pos = atomicAdd(&hist[c], run);
      for (int r = 0; r < run; ++r)
        if (pos + r < capacity) {
          plan[4 + 2 * (pos + r)] = s;
          plan[5 + 2 * (pos + r)] = qt + r;
        }
      qt += run;
    }
  }
}

}  // namespace attn
