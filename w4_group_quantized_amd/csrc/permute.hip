// Token permutation by expert: histogram, exclusive scan, stable scatter and
// row gather, so that each expert's tokens form one contiguous segment for
// the grouped FFN (xdnf.cn/news/329730 §3.2: tokens that chose the same
// expert are gathered and computed together).
//
// Flat index f = t*k + j.  Segment e holds the f with idx[f] = e in
// increasing f, which makes offsets, perm_src and inv_pos unique.
//
//   count:   one block per chunk of kPermChunk entries, LDS histogram
//   scan:    one block: per-expert totals -> offsets, per-chunk bases, the
//            chunks of each expert split over 1024 / E threads
//   scatter: one wave per chunk; ranks within a wave by matching expert ids
//            through ballots over their bits, in flat order
//   gather:  x_perm[r] = x[perm_src[r] / k], 16-byte copies (optional: the
//            FFN can read the rows of x through perm_src instead)
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxExperts = 1024;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t *__restrict__ idx, int N,
                                                         int E, int32_t *__restrict__ counts) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int f = blockIdx.x * kPermChunk + threadIdx.x;
  if (f < N) atomicAdd(&hist[clamp_expert(idx[f], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads.  Thread (p, e) = (tid / Ep, tid % Ep), Ep the
// power of two >= E: the P = 1024 / Ep threads of expert e each sum the
// counts of a contiguous range of chunks; their partial sums give each
// thread the expert's total and the count before its range, the totals are
// scanned over experts (offsets), and each thread then writes the running
// bases of its chunks.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t *__restrict__ counts,
                                                         int nchunks, int E, int Ep,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ bases) {
  __shared__ int part[1024];
  __shared__ int s_off[kMaxExperts];
  __shared__ int scratch[16];
  const int tid = threadIdx.x;
  const int P = 1024 / Ep;
  const int e = tid % Ep, pp = tid / Ep;
  const int c0 = (int)((int64_t)pp * nchunks / P), c1 = (int)((int64_t)(pp + 1) * nchunks / P);
  int sum = 0;
  if (e < E) {
    // eight independent loads in flight per round
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = counts[(size_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
    for (; c < c1; ++c) sum += counts[(size_t)c * E + e];
  }
  part[tid] = sum;
  __syncthreads();
  int pre = 0, tot = 0;
  if (e < E)
    for (int q = 0; q < P; ++q) {
      const int v = part[q * Ep + e];
      pre += q < pp ? v : 0;
      tot += v;
    }
  int total;
  const int excl = block_excl_scan(pp == 0 && e < E ? tot : 0, scratch, &total);
  if (pp == 0 && e < E) {
    s_off[e] = excl;
    offsets[e] = excl;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  if (e < E) {
    int run = s_off[e] + pre;
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = counts[(size_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bases[(size_t)(c + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; c < c1; ++c) {
      const int v = counts[(size_t)c * E + e];
      bases[(size_t)c * E + e] = run;
      run += v;
    }
  }
}

// One wave per chunk.
__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t *__restrict__ idx, int N,
                                                          int E, const int32_t *__restrict__ bases,
                                                          int32_t *__restrict__ perm_src,
                                                          int32_t *__restrict__ inv_pos) {
  __shared__ int run[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) run[e] = bases[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int sub = 0; sub < kPermChunk / kWave; ++sub) {
    const int f = blockIdx.x * kPermChunk + sub * kWave + lane;
    const bool valid = f < N;
    const int e = valid ? clamp_expert(idx[f], E) : E;   // E marks an empty lane
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {   // ids 0..1024 fit in 11 bits
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int base = valid ? run[e] : 0;
    const int r = base + rank;
    if (valid && (same & below) == 0ull) run[e] = base + __popcll(same);
    if (valid) {
      perm_src[r] = f;
      inv_pos[f] = r;
    }
    __syncthreads();
  }
}

// 4 permuted rows per block, one wave per row.
__global__ __launch_bounds__(256) void perm_gather_kernel(const f16 *__restrict__ x,
                                                          const int32_t *__restrict__ perm_src,
                                                          int N, int k, int T, int H,
                                                          f16 *__restrict__ x_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= N) return;
  int t = perm_src[r] / k;
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)t * H);
  u32x4 *dst = reinterpret_cast<u32x4 *>(x_perm + (size_t)r * H);
  for (int c = lane; c < H / 8; c += kWave) dst[c] = src[c];
}

hipError_t launch_permute(const moe_layer &L, const uint16_t *x, const int32_t *idx, int32_t T,
                          int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                          uint16_t *x_perm, int32_t *counts, int32_t *bases, hipStream_t st) {
  const int E = L.num_experts, k = L.top_k;
  const int N = T * k;
  const int nchunks = (N + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(256), 0, st, idx, N, E, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int Ep = 1;
  while (Ep < E) Ep *= 2;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, counts, nchunks, E, Ep,
                     offsets, bases);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(64), 0, st, idx, N, E, bases,
                     perm_src, inv_pos);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (!x_perm) return hipSuccess;
  return launch_gather(L, x, perm_src, T, x_perm, st);
}

hipError_t launch_gather(const moe_layer &L, const uint16_t *x, const int32_t *perm_src, int32_t T,
                         uint16_t *x_perm, hipStream_t st) {
  const int k = L.top_k, H = L.hidden;
  const int N = T * k;
  hipLaunchKernelGGL(perm_gather_kernel, dim3((N + 3) / 4), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(x), perm_src, N, k, T, H,
                     reinterpret_cast<f16 *>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
