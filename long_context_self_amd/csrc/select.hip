// Verification-guided top-k selection for gfx950.
//
// What is computed
//  * Vegas page, "Core claim" / "What carries the argument": the logits of the
//    first draft row and the bonus row are combined across the query heads and
//    the k prefix positions with the largest combined score are kept.
//  * Sparse Glimpse page, "Core claim": sink + recent + top-ranked history, one
//    set per head (here per KV head, scored over the heads of its group).
//  * SSV page, NSA block selection: a block scores the max of its positions.
//  Score of position p: sigma_p = sum over the set's heads h (ascending) of
//  (l[h,row0,p] + l[h,row1,p]) in that fixed fp32 order; -0 is taken as +0.  Ties
//  at the k-th place go to the smaller index; output is ascending.
//
// How
//  * score_kernel streams the two logit rows of every head once (the only HBM-
//    sized read), writes an order-preserving uint32 key per item, and builds a
//    4096-bin histogram of the top 12 key bits in LDS, flushed with one global
//    atomic per non-empty bin.
//  * collect_kernel finds the bin that holds the k-th item, counts items above it
//    per 4096-item chunk and appends the bin's items as 44-bit composites
//    (20 low key bits, then the complemented index) to a candidate list.
//  * finalize_kernel (one workgroup per set) radix-selects the exact boundary
//    composite among the candidates in four 11-bit LDS passes, then turns the
//    per-chunk counts into output offsets.
//  * emit_kernel rescans each chunk and writes the kept items in ascending order
//    with a workgroup prefix sum.
//  No transcendental function and no multiply is involved, so the result is
//  bit-identical to the same rule evaluated on the CPU in the same order.
#include "lcs_internal.h"

namespace lcs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kItemBits = 24;                       // items < 2^24
constexpr uint32_t kItemMask = (1u << kItemBits) - 1;

__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.f) u = 0u;                             // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int item) {
  return ((uint64_t)(key & 0xFFFFFu) << kItemBits) | (uint64_t)(kItemMask - (uint32_t)item);
}

struct Win {
  int L, n, lo, hi;
  bool all;
};

// Items, pool [lo, hi) and the keep-everything case for sequence b.
__device__ __forceinline__ Win window(const SelArgs& a, int b) {
  Win w;
  w.L = min(max(a.prefix_len[b], 0), a.max_len);
  if (a.mode == LCS_SEL_BLOCK) {
    const int bs = 1 << a.lg_bs;
    w.n = (w.L + bs - 1) >> a.lg_bs;
    w.lo = (a.n_sink + bs - 1) >> a.lg_bs;
    w.hi = (a.n_recent > 0) ? ((w.L - a.n_recent) >= 0 ? (w.L - a.n_recent) >> a.lg_bs : -1) : w.n;
    w.all = (w.lo >= w.hi) || (w.hi - w.lo <= a.top_k);
  } else {
    w.n = w.L;
    w.lo = a.n_sink;
    w.hi = w.L - a.n_recent;
    w.all = w.L <= a.n_sink + a.top_k + a.n_recent;
  }
  return w;
}

__global__ void zero_kernel(SelArgs a, int NS) {
  const int n = NS * kHistBins;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) a.hist[i] = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < NS; i += gridDim.x * blockDim.x) a.cand_count[i] = 0;
}

__global__ void __launch_bounds__(256) score_kernel(SelArgs a) {
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const int s = set - b * a.n_sets;
  const Win w = window(a, b);
  if (w.all || a.top_k == 0) return;
  const int p0 = blockIdx.x * kSelChunk;
  if (p0 >= w.L) return;
  const int tid = threadIdx.x;
  const int h0 = (a.mode == LCS_SEL_SHARED) ? 0 : s * a.G;
  const int nh = (a.mode == LCS_SEL_SHARED) ? a.Hq : a.G;

  __shared__ uint32_t lh[kHistBins];
  __shared__ uint32_t bm[kSelChunk / 4];
  for (int i = tid; i < kHistBins; i += 256) lh[i] = 0;
  if (a.mode == LCS_SEL_BLOCK)
    for (int i = tid; i < kSelChunk / 4; i += 256) bm[i] = 0;
  __syncthreads();

  // sigma for positions p0 + it*1024 + 4*tid + [0, 4)
  f32x4 acc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* base = a.logits + (size_t)b * a.Hq * 2 * a.ld;
  const bool fast = a.vec4 && (p0 + kSelChunk <= w.L);
  if (fast) {
#pragma unroll 4
    for (int hh = 0; hh < nh; ++hh) {
      const float* r0 = base + (size_t)(h0 + hh) * 2 * a.ld + p0 + 4 * tid;
      const float* r1 = r0 + a.ld;
      f32x4 x0[4], x1[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        x0[it] = *reinterpret_cast<const f32x4*>(r0 + it * 1024);
        x1[it] = *reinterpret_cast<const f32x4*>(r1 + it * 1024);
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) acc[it] = acc[it] + (x0[it] + x1[it]);
    }
  } else {
    for (int hh = 0; hh < nh; ++hh) {
      const float* r0 = base + (size_t)(h0 + hh) * 2 * a.ld;
      const float* r1 = r0 + a.ld;
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = p0 + it * 1024 + 4 * tid + k;
          if (p < w.L) acc[it][k] = acc[it][k] + (r0[p] + r1[p]);
        }
    }
  }

  uint32_t* keys = a.keys + (size_t)set * a.item_cap;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int p = p0 + it * 1024 + 4 * tid;
    uint32_t kk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) kk[k] = f2key(acc[it][k]);
    if (a.mode != LCS_SEL_BLOCK) {
      if (p + 3 < w.L) {
        *reinterpret_cast<u32x4*>(keys + p) = u32x4{kk[0], kk[1], kk[2], kk[3]};
      } else {
        for (int k = 0; k < 4; ++k)
          if (p + k < w.L) keys[p + k] = kk[k];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (p + k >= w.lo && p + k < w.hi) atomicAdd(&lh[kk[k] >> 20], 1u);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (p + k < w.L) atomicMax(&bm[(it * 1024 + 4 * tid + k) >> a.lg_bs], kk[k]);
    }
  }
  __syncthreads();
  if (a.mode == LCS_SEL_BLOCK) {
    const int nbc = kSelChunk >> a.lg_bs;
    const int c0 = p0 >> a.lg_bs;
    for (int cl = tid; cl < nbc; cl += 256) {
      const int c = c0 + cl;
      if (c < w.n) {
        keys[c] = bm[cl];
        if (c >= w.lo && c < w.hi) atomicAdd(&lh[bm[cl] >> 20], 1u);
      }
    }
    __syncthreads();
  }
  uint32_t* gh = a.hist + (size_t)set * kHistBins;
  for (int i = tid; i < kHistBins; i += 256)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Threshold bin of set `set` from its histogram: the bin holding the k-th largest item.
__device__ void find_bin(const SelArgs& a, int set, uint32_t* ts, int& bin_out, uint32_t& above_out,
                         int* sh_bin, uint32_t* sh_above) {
  const int tid = threadIdx.x;
  const uint32_t* h = a.hist + (size_t)set * kHistBins;
  uint32_t c = 0;
  for (int e = 0; e < 16; ++e) c += h[16 * tid + e];
  // inclusive scan from the top: ts[t] = sum over threads t' >= t
  ts[tid] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = (tid + off < 256) ? ts[tid + off] : 0;
    __syncthreads();
    ts[tid] += v;
    __syncthreads();
  }
  const uint32_t K = (uint32_t)a.top_k;
  const uint32_t above_t = ts[tid] - c;             // items in bins above this thread's range
  if (above_t < K && above_t + c >= K) {
    uint32_t cum = above_t;
    for (int bin = 16 * tid + 15; bin >= 16 * tid; --bin) {
      if (cum + h[bin] >= K) {
        *sh_bin = bin;
        *sh_above = cum;
        break;
      }
      cum += h[bin];
    }
  }
  __syncthreads();
  bin_out = *sh_bin;
  above_out = *sh_above;
}

__global__ void __launch_bounds__(256) collect_kernel(SelArgs a) {
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const Win w = window(a, b);
  if (w.all || a.top_k == 0) return;
  const int tid = threadIdx.x;
  __shared__ uint32_t ts[256];
  __shared__ int sh_bin;
  __shared__ uint32_t sh_above;
  __shared__ uint64_t lq[kSelChunk];
  __shared__ uint32_t lqn, lqbase, nab;
  if (tid == 0) {
    sh_bin = 0;
    sh_above = 0;
    lqn = 0;
    nab = 0;
  }
  __syncthreads();
  int bin;
  uint32_t above;
  find_bin(a, set, ts, bin, above, &sh_bin, &sh_above);
  if (blockIdx.x == 0 && tid == 0) {
    a.thr[(size_t)set * 2 + 0] = (uint64_t)bin;
    a.thr[(size_t)set * 2 + 1] = (uint64_t)above;
  }
  const int i0 = blockIdx.x * kSelChunk;
  const int lo = max(w.lo, i0), hi = min(w.hi, i0 + kSelChunk);
  const uint32_t* keys = a.keys + (size_t)set * a.item_cap;
  uint32_t my_above = 0;
  for (int it = lo + tid; it < hi; it += 256) {
    const uint32_t key = keys[it];
    const int dg = (int)(key >> 20);
    if (dg > bin) {
      ++my_above;
    } else if (dg == bin) {
      const uint32_t slot = atomicAdd(&lqn, 1u);
      lq[slot] = composite(key, it);
    }
  }
  atomicAdd(&nab, my_above);
  __syncthreads();
  if (tid == 0) {
    lqbase = lqn ? atomicAdd(&a.cand_count[set], lqn) : 0;
    a.chunk_above[(size_t)set * a.n_chunks + blockIdx.x] = nab;
  }
  __syncthreads();
  uint64_t* cand = a.cand + (size_t)set * a.item_cap;
  for (uint32_t e = tid; e < lqn; e += 256)
    if (lqbase + e < (uint32_t)a.item_cap) cand[lqbase + e] = lq[e];
}

__global__ void __launch_bounds__(1024) finalize_kernel(SelArgs a) {
  const int set = blockIdx.x;
  const int b = set / a.n_sets;
  const Win w = window(a, b);
  if (w.all || a.top_k == 0) return;
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cc[kHistBins];
  __shared__ uint64_t sh_prefix, sh_mask;
  __shared__ uint32_t sh_rem;
  const uint32_t above = (uint32_t)a.thr[(size_t)set * 2 + 1];
  const uint32_t need = (uint32_t)a.top_k - above;
  const int n_c = min((int)a.cand_count[set], a.item_cap);
  const uint64_t* cand = a.cand + (size_t)set * a.item_cap;
  if (tid == 0) {
    sh_prefix = 0;
    sh_mask = 0;
    sh_rem = need;
  }
  __syncthreads();
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 33 - 11 * pass;
    for (int i = tid; i < 2048; i += 1024) hist[i] = 0;
    __syncthreads();
    const uint64_t prefix = sh_prefix, mask = sh_mask;
    for (int e = tid; e < n_c; e += 1024) {
      const uint64_t c = cand[e];
      if ((c & mask) == prefix) atomicAdd(&hist[(c >> shift) & 2047u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t rem = sh_rem;
      int d = 2047;
      for (; d > 0; --d) {
        if (hist[d] >= rem) break;
        rem -= hist[d];
      }
      sh_rem = rem;
      sh_prefix = prefix | ((uint64_t)d << shift);
      sh_mask = mask | ((uint64_t)2047u << shift);
    }
    __syncthreads();
  }
  const uint64_t cstar = sh_prefix;
  // per-chunk kept counts -> exclusive offsets (after the sink window)
  for (int c = tid; c < a.n_chunks; c += 1024) cc[c] = a.chunk_above[(size_t)set * a.n_chunks + c];
  __syncthreads();
  for (int e = tid; e < n_c; e += 1024) {
    const uint64_t c = cand[e];
    if (c >= cstar) {
      const int item = (int)(kItemMask - (uint32_t)(c & kItemMask));
      atomicAdd(&cc[item / kSelChunk], 1u);
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = (uint32_t)w.lo;
    uint32_t* off = a.chunk_off + (size_t)set * a.n_chunks;
    for (int c = 0; c < a.n_chunks; ++c) {
      off[c] = run;
      run += cc[c];
    }
    a.thr[(size_t)set * 2 + 1] = cstar;
  }
}

__global__ void __launch_bounds__(256) emit_kernel(SelArgs a) {
  const int set = blockIdx.y;
  const int b = set / a.n_sets;
  const Win w = window(a, b);
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * kSelChunk;
  int32_t* out = a.indices + (size_t)set * a.cap;
  if (w.all) {
    for (int it = i0 + tid; it < min(w.n, i0 + kSelChunk); it += 256)
      if (it < a.cap) out[it] = it;
    if (blockIdx.x == 0 && tid == 0) a.counts[set] = min(w.n, a.cap);
    return;
  }
  const int K = a.top_k;
  const int bin = (K > 0) ? (int)a.thr[(size_t)set * 2 + 0] : 0;
  const uint64_t cstar = (K > 0) ? a.thr[(size_t)set * 2 + 1] : ~0ull;
  const uint32_t* keys = a.keys + (size_t)set * a.item_cap;
  __shared__ uint32_t ts[256];
  // thread t owns items [i0 + 16t, i0 + 16t + 16)
  uint32_t flags = 0;
  int cnt = 0;
  for (int e = 0; e < 16; ++e) {
    const int it = i0 + 16 * tid + e;
    if (it >= w.lo && it < w.hi && K > 0) {
      const uint32_t key = keys[it];
      const int dg = (int)(key >> 20);
      const bool keep = dg > bin || (dg == bin && composite(key, it) >= cstar);
      if (keep) {
        flags |= 1u << e;
        ++cnt;
      }
    }
  }
  ts[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = (tid >= off) ? ts[tid - off] : 0;
    __syncthreads();
    ts[tid] += v;
    __syncthreads();
  }
  uint32_t pos = ((K > 0) ? a.chunk_off[(size_t)set * a.n_chunks + blockIdx.x] : (uint32_t)w.lo) + ts[tid] - cnt;
  for (int e = 0; e < 16; ++e) {
    const int it = i0 + 16 * tid + e;
    if (it >= w.n) break;
    if (it < w.lo) {
      if (it < a.cap) out[it] = it;
    } else if (it >= w.hi) {
      const int o = w.lo + K + (it - w.hi);
      if (o < a.cap) out[o] = it;
    } else if (flags & (1u << e)) {
      if ((int)pos < a.cap) out[pos] = it;
      ++pos;
    }
  }
  if (blockIdx.x == 0 && tid == 0) a.counts[set] = min(w.lo + K + (w.n - w.hi), a.cap);
}

}  // namespace

SelPlan select_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t mode, int32_t max_len,
                    int32_t block_size) {
  SelPlan p{};
  p.n_sets = (mode == LCS_SEL_SHARED) ? 1 : Hkv;
  const size_t NS = (size_t)B * p.n_sets;
  long long items = max_len;
  if (mode == LCS_SEL_BLOCK) items = (max_len + block_size - 1) / block_size;
  if (items < 1) items = 1;
  p.item_cap = (int32_t)align_up((size_t)items, 4);
  p.n_chunks = (int32_t)((items + kSelChunk - 1) / kSelChunk);
  p.n_pos_chunks = (int32_t)(((long long)(max_len > 0 ? max_len : 1) + kSelChunk - 1) / kSelChunk);
  p.keys_bytes = align_up(NS * p.item_cap * 4, 256);
  p.hist_bytes = align_up(NS * kHistBins * 4, 256);
  p.cc_bytes = align_up(NS * 4, 256);
  p.cand_bytes = align_up(NS * p.item_cap * 8, 256);
  p.ca_bytes = align_up(NS * p.n_chunks * 4, 256);
  p.co_bytes = align_up(NS * p.n_chunks * 4, 256);
  p.thr_bytes = align_up(NS * 2 * 8, 256);
  p.total_bytes = p.keys_bytes + p.hist_bytes + p.cc_bytes + p.cand_bytes + p.ca_bytes +
                  p.co_bytes + p.thr_bytes;
  return p;
}

hipError_t select_launch(const SelPlan& p, SelArgs a, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  a.keys = reinterpret_cast<uint32_t*>(ws); ws += p.keys_bytes;
  a.hist = reinterpret_cast<uint32_t*>(ws); ws += p.hist_bytes;
  a.cand_count = reinterpret_cast<uint32_t*>(ws); ws += p.cc_bytes;
  a.cand = reinterpret_cast<uint64_t*>(ws); ws += p.cand_bytes;
  a.chunk_above = reinterpret_cast<uint32_t*>(ws); ws += p.ca_bytes;
  a.chunk_off = reinterpret_cast<uint32_t*>(ws); ws += p.co_bytes;
  a.thr = reinterpret_cast<uint64_t*>(ws);
  a.n_sets = p.n_sets;
  a.item_cap = p.item_cap;
  a.n_chunks = p.n_chunks;
  a.n_pos_chunks = p.n_pos_chunks;
  const int NS = a.B * p.n_sets;
  hipLaunchKernelGGL(zero_kernel, dim3(min(1024, (NS * kHistBins + 255) / 256)), dim3(256), 0, stream, a, NS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_kernel, dim3(p.n_pos_chunks, NS), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(collect_kernel, dim3(p.n_chunks, NS), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(NS), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_kernel, dim3(p.n_chunks, NS), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lcs
