// dispatch.hip -- deterministic counting sort of routed pairs by local
// expert, and of tokens by the wave after which they can be combined.
//
// 10100.com commentary (section on batch-invariant and deterministic
// operators): the deterministic kernels pre-sort instead of letting
// unordered atomics decide positions.  Here no position is ever taken from
// an atomic counter: every pair's row is a pure function of topk_idx.
//
//   1. count  : per 64-token chunk (one wavefront) build, in LDS, a bitmask
//               per group (local expert, ready-wave slot) of the chunk's
//               tokens in that group.  Bit OR is order-independent, so the
//               masks are deterministic.
//   2. scan   : per group (one wavefront), exclusive scan of popcounts over
//               chunks in ascending chunk order; then exclusive scan of group
//               totals.
//   3. scatter: a token's row inside its group is the group start + the
//               chunk's base + the number of lower lanes in the same mask,
//               so rows within a group follow ascending token id.
#include "moe_internal.h"
#include "route_topk.h"

namespace moe {
namespace {

constexpr int kChunksPerBlock = 4;  // 4 wavefronts of 64 tokens

__global__ __launch_bounds__(256) void dispatch_count_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int e_begin, int E_local, int G,
    int ngroups, unsigned long long* __restrict__ masks, int32_t* __restrict__ ready_wave) {
  extern __shared__ unsigned long long smask[];  // [kChunksPerBlock][ngroups]
  const int wave = wave_id(), lane = lane_id();
  for (int i = threadIdx.x; i < kChunksPerBlock * ngroups; i += blockDim.x) smask[i] = 0ull;
  __syncthreads();
  const int chunk = blockIdx.x * kChunksPerBlock + wave;
  const int t = chunk * kWave + lane;
  unsigned long long* my = smask + wave * ngroups;
  if (t < T) {
    int ready = -1;
    for (int j = 0; j < k; ++j) {
      const int le = topk_idx[static_cast<size_t>(t) * k + j] - e_begin;
      if (le >= 0 && le < E_local) {
        atomicOr(&my[le], 1ull << lane);
        ready = max(ready, le / G);
      }
    }
    atomicOr(&my[E_local + 1 + ready], 1ull << lane);
    ready_wave[t] = ready;
  }
  __syncthreads();
  const int nchunks = (T + kWave - 1) / kWave;
  for (int i = threadIdx.x; i < kChunksPerBlock * ngroups; i += blockDim.x) {
    const int c = blockIdx.x * kChunksPerBlock + i / ngroups;
    if (c < nchunks) masks[static_cast<size_t>(c) * ngroups + i % ngroups] = smask[i];
  }
}

// One block of 1024 threads; wavefront w owns groups w, w + 16, ...
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const unsigned long long* __restrict__ masks, int nchunks, int ngroups, int E_local,
    int32_t* __restrict__ bases, int32_t* __restrict__ group_off, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ err, int32_t* __restrict__ ctr, int n_ctr) {
  extern __shared__ int32_t stot[];  // [ngroups]
  if (threadIdx.x == 0) *err = 0;  // a new layer call starts with a clean error word
  // the expert-wave kernel's counters start the layer call at zero (that
  // kernel clears them again when it ends, for back-to-back FFN calls)
  for (int i = threadIdx.x; i < n_ctr; i += blockDim.x) ctr[i] = 0;
  // one wavefront per group: lanes take 64 chunks at a time, an exclusive
  // prefix sum of their popcounts (shuffles) gives the chunks' bases, and
  // the running total carries over to the next 64 chunks
  const int lane = lane_id(), nwaves = blockDim.x / kWave;
  for (int g = wave_id(); g < ngroups; g += nwaves) {
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kWave) {
      const int c = c0 + lane;
      const int v = c < nchunks ? __popcll(masks[static_cast<size_t>(c) * ngroups + g]) : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        incl += lane >= off ? o : 0;
      }
      if (c < nchunks) bases[static_cast<size_t>(c) * ngroups + g] = carry + incl - v;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) stot[g] = carry;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // expert groups and ready-wave groups are two separate sorted orders
    int run = 0;
    for (int g = 0; g < E_local; ++g) {
      group_off[g] = run;
      offsets[g] = run;
      counts[g] = stot[g];
      run += stot[g];
    }
    group_off[E_local] = run;
    offsets[E_local] = run;
    run = 0;
    for (int g = E_local; g < ngroups; ++g) {
      group_off[g + 1] = run;
      run += stot[g];
    }
    // group_off[E_local + 1 + s] = start of ready slot s; last = T
    group_off[ngroups + 1] = run;
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int e_begin, int E_local, int ngroups,
    const unsigned long long* __restrict__ masks, const int32_t* __restrict__ bases,
    const int32_t* __restrict__ group_off, const int32_t* __restrict__ ready_wave,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ ready_list) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int chunk = t / kWave, lane = t % kWave;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const size_t crow = static_cast<size_t>(chunk) * ngroups;
  for (int j = 0; j < k; ++j) {
    const int le = topk_idx[static_cast<size_t>(t) * k + j] - e_begin;
    int32_t row = -1;
    if (le >= 0 && le < E_local) {
      row = group_off[le] + bases[crow + le] + __popcll(masks[crow + le] & below);
      sorted_token[row] = t;
    }
    pair_pos[static_cast<size_t>(t) * k + j] = row;
  }
  const int slot = ready_wave[t] + 1;
  const int g = E_local + slot;
  ready_list[group_off[E_local + 1 + slot] + bases[crow + g] + __popcll(masks[crow + g] & below)] = t;
}

// The three steps above in one workgroup of 1024 threads, for batches of at
// most kSmallChunks chunks (T <= 1024: a chunk per wavefront, a token per
// thread): masks, bases and group starts stay in LDS and the launches
// between the steps disappear (decode: 19 -> 11 us per dispatch).  The
// arithmetic is the same as the three kernels', so every output is the
// same.  Larger batches keep the three kernels: one workgroup then costs
// more than the launches it saves (T = 4096: 27 us against 15-19 us).
constexpr int kSmallChunks = 16;

// The router's selection for the batch first (TOPK, route-and-dispatch
// of small batches): one wavefront per token over the partial logits, the
// same instructions as moe_route's top-k kernel (route_topk.h); topk_idx
// and topk_w are written to global memory and read back below by the whole
// workgroup after a barrier.
struct SmallTopk {
  const float* partial;
  int splits;
  const float* bias;
  int E;
  float* topk_w;
  float* logits;
};

template <bool TOPK>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    const int32_t* topk_idx, int T, int k, int e_begin, int E_local, int G, int ngroups,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ group_off,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pair_pos, int32_t* __restrict__ ready_wave,
    int32_t* __restrict__ ready_list, int32_t* __restrict__ err, int32_t* __restrict__ ctr, int n_ctr,
    SmallTopk tk) {
  extern __shared__ unsigned long long smask[];  // [nchunks][ngroups], then the int32 tables
  const int nchunks = (T + kWave - 1) / kWave;
  int32_t* sbase = reinterpret_cast<int32_t*>(smask + static_cast<size_t>(nchunks) * ngroups);  // [nchunks][ngroups]
  int32_t* sgoff = sbase + nchunks * ngroups;                                                   // [ngroups + 2]
  int32_t* stot = sgoff + ngroups + 2;                                                          // [ngroups]
  const int wave = wave_id(), lane = lane_id(), nwaves = blockDim.x / kWave;
  if constexpr (TOPK) {
    for (int t = wave; t < T; t += nwaves)
      topk_token(tk.partial, tk.splits, tk.bias, T, tk.E, k, t, const_cast<int32_t*>(topk_idx), tk.topk_w,
                 tk.logits);
    __syncthreads();
  }
  if (threadIdx.x == 0) *err = 0;  // a new layer call starts with a clean error word
  for (int i = threadIdx.x; i < n_ctr; i += blockDim.x) ctr[i] = 0;
  for (int i = threadIdx.x; i < nchunks * ngroups; i += blockDim.x) smask[i] = 0ull;
  __syncthreads();
  // 1. count: wavefront w takes chunks w, w + 16, ...
  for (int c = wave; c < nchunks; c += nwaves) {
    const int t = c * kWave + lane;
    unsigned long long* my = smask + static_cast<size_t>(c) * ngroups;
    if (t < T) {
      int ready = -1;
      for (int j = 0; j < k; ++j) {
        const int le = topk_idx[static_cast<size_t>(t) * k + j] - e_begin;
        if (le >= 0 && le < E_local) {
          atomicOr(&my[le], 1ull << lane);
          ready = max(ready, le / G);
        }
      }
      atomicOr(&my[E_local + 1 + ready], 1ull << lane);
      ready_wave[t] = ready;
    }
  }
  __syncthreads();
  // 2. scan: one wavefront per group, the chunks on its lanes (nchunks <= 64)
  for (int g = wave; g < ngroups; g += nwaves) {
    const int v = lane < nchunks ? __popcll(smask[static_cast<size_t>(lane) * ngroups + g]) : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      incl += lane >= off ? o : 0;
    }
    if (lane < nchunks) sbase[lane * ngroups + g] = incl - v;
    if (lane == kWave - 1) stot[g] = incl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int g = 0; g < E_local; ++g) {
      sgoff[g] = run;
      offsets[g] = run;
      counts[g] = stot[g];
      run += stot[g];
    }
    sgoff[E_local] = run;
    offsets[E_local] = run;
    run = 0;
    for (int g = E_local; g < ngroups; ++g) {
      sgoff[g + 1] = run;
      run += stot[g];
    }
    sgoff[ngroups + 1] = run;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ngroups + 2; i += blockDim.x) group_off[i] = sgoff[i];
  // 3. scatter: one thread per token
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    const int c = t / kWave, l = t % kWave;
    const unsigned long long below = (l == 0) ? 0ull : (~0ull >> (kWave - l));
    const int crow = c * ngroups;
    for (int j = 0; j < k; ++j) {
      const int le = topk_idx[static_cast<size_t>(t) * k + j] - e_begin;
      int32_t row = -1;
      if (le >= 0 && le < E_local) {
        row = sgoff[le] + sbase[crow + le] + __popcll(smask[crow + le] & below);
        sorted_token[row] = t;
      }
      pair_pos[static_cast<size_t>(t) * k + j] = row;
    }
    const int slot = ready_wave[t] + 1;
    const int g = E_local + slot;
    ready_list[sgoff[E_local + 1 + slot] + sbase[crow + g] + __popcll(smask[crow + g] & below)] = t;
  }
}

size_t dispatch_small_lds(const WsLayout& L) {
  return static_cast<size_t>(L.nchunks) * L.ngroups * 12 + (2 * static_cast<size_t>(L.ngroups) + 2) * 4;
}

bool dispatch_uses_small(const moe_problem_t& p, const WsLayout& L) {
  return p.T > 0 && L.nchunks <= kSmallChunks && dispatch_small_lds(L) <= 64 * 1024;
}

}  // namespace

bool route_dispatch_fuses(const moe_problem_t& p, const WsLayout& L) {
  return p.T <= kFusedTopkMaxTokens && dispatch_uses_small(p, L);
}

hipError_t launch_dispatch_with_topk(const moe_problem_t& p, const WsLayout& L, const float* partial,
                                     const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                                     int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                                     int32_t* pair_pos, int32_t* ready_wave, char* ws, hipStream_t s) {
  SmallTopk tk{partial, router_splits(p.d, p.E_global, p.x_dtype == MOE_BF16), bias, p.E_global, topk_w, logits};
  dispatch_small_kernel<true><<<1, 1024, dispatch_small_lds(L), s>>>(
      topk_idx, p.T, p.k, p.e_begin, p.E_local, p.experts_per_wave, L.ngroups, counts, offsets,
      reinterpret_cast<int32_t*>(ws + L.group_off), sorted_token, pair_pos, ready_wave,
      reinterpret_cast<int32_t*>(ws + L.ready_list), reinterpret_cast<int32_t*>(ws + L.err),
      reinterpret_cast<int32_t*>(ws + L.sync), static_cast<int>(L.sync_words), tk);
  return hipGetLastError();
}

hipError_t launch_dispatch(const moe_problem_t& p, const WsLayout& L, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                           int32_t* pair_pos, int32_t* ready_wave, char* ws, hipStream_t s) {
  auto* masks = reinterpret_cast<unsigned long long*>(ws + L.masks);
  auto* bases = reinterpret_cast<int32_t*>(ws + L.bases);
  auto* group_off = reinterpret_cast<int32_t*>(ws + L.group_off);
  auto* ready_list = reinterpret_cast<int32_t*>(ws + L.ready_list);
  const int blocks = (L.nchunks + kChunksPerBlock - 1) / kChunksPerBlock;
  if (dispatch_uses_small(p, L)) {
    dispatch_small_kernel<false><<<1, 1024, dispatch_small_lds(L), s>>>(
        topk_idx, p.T, p.k, p.e_begin, p.E_local, p.experts_per_wave, L.ngroups, counts, offsets, group_off,
        sorted_token, pair_pos, ready_wave, ready_list, reinterpret_cast<int32_t*>(ws + L.err),
        reinterpret_cast<int32_t*>(ws + L.sync), static_cast<int>(L.sync_words), SmallTopk{});
    return hipGetLastError();
  }
  if (p.T > 0) {
    dispatch_count_kernel<<<blocks, 256, kChunksPerBlock * L.ngroups * sizeof(unsigned long long), s>>>(
        topk_idx, p.T, p.k, p.e_begin, p.E_local, p.experts_per_wave, L.ngroups, masks, ready_wave);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dispatch_scan_kernel<<<1, 1024, L.ngroups * sizeof(int32_t), s>>>(
      masks, L.nchunks, L.ngroups, p.E_local, bases, group_off, counts, offsets,
      reinterpret_cast<int32_t*>(ws + L.err), reinterpret_cast<int32_t*>(ws + L.sync),
      static_cast<int>(L.sync_words));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.T == 0) return e;
  dispatch_scatter_kernel<<<(p.T + 255) / 256, 256, 0, s>>>(
      topk_idx, p.T, p.k, p.e_begin, p.E_local, L.ngroups, masks, bases, group_off, ready_wave,
      sorted_token, pair_pos, ready_list);
  return hipGetLastError();
}

}  // namespace moe
