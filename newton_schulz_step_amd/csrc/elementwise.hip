// Streaming kernels of the Muon step (gfx950): momentum with per-problem sums of
// squares, the Frobenius normalisation into the iteration's storage type, AdamW,
// and bit-exact batched copies for packing.
//
// All of these are bound by HBM bandwidth: consecutive threads touch consecutive
// vectors, each thread moves a few elements in one pass (no loops), and
// reductions run in a fixed order (wave butterflies, then a fixed sum over
// waves, then a fixed-order float64 sum over blocks) so results do not depend on
// scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace muon {

// ---------------------------------------------------------------------------
// per-problem descriptors: block y of a launch writes the problems of entry y of
// its chunk (split blocks of a matrix are consecutive problems of one group)

struct DescChunk {
  EntryRec e[kDescChunk];
};

__global__ __launch_bounds__(256) void expand_desc_kernel(DescChunk c, ProblemDesc* out) {
  const EntryRec r = c.e[blockIdx.y];
  const int64_t nblk = r.nblk_t >> 1;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; b < nblk;
       b += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t bi = b / r.ncb;
    const int64_t first = bi * r.rstep + (b - bi * r.ncb) * r.cstep;   // matrix flat index of element 0
    ProblemDesc d;
    d.src_off = r.offset + first;
    d.p_base = r.p0 + first;
    d.lo = min(max(r.lo - first, int64_t(0)), r.span);
    d.hi = min(max(r.hi - first, int64_t(0)), r.span);
    d.transposed = r.nblk_t & 1;
    d.ld = r.ld;
    d.w = r.w;
    d.pad = 0;
    out[r.first + b] = d;
  }
}

hipError_t launch_expand_desc(const EntryRec* entries, int n, ProblemDesc* out, hipStream_t s) {
  static_assert(sizeof(ProblemDesc) == kProblemDescBytes, "descriptor size used by the workspace layout");
  for (int i = 0; i < n; i += kDescChunk) {
    const int cnt = n - i < kDescChunk ? n - i : kDescChunk;
    DescChunk c;
    int64_t most = 1;
    for (int k = 0; k < kDescChunk; ++k) c.e[k] = k < cnt ? entries[i + k] : EntryRec{};
    for (int k = 0; k < cnt; ++k) most = max(most, static_cast<int64_t>(entries[i + k].nblk_t >> 1));
    const int64_t gx = min((most + 255) / 256, int64_t(256));
    hipLaunchKernelGGL(expand_desc_kernel, dim3(static_cast<unsigned>(gx), cnt), dim3(256), 0, s, c, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// momentum (DeepSpeed-Muon article, "什么是 Muon 优化器？": momentum first) and the
// sum of squares that the Frobenius normalisation needs

// One block of kMomThreads threads updates kMomChunk consecutive elements of one
// problem, four per thread (one 16-byte momentum vector): many small blocks keep
// the most reads and writes in flight across the HBM channels. A problem's
// elements are taken in its stored row-major order; a block narrower than its
// matrix (a column block) steps from the end of one of its rows to the next
// row's start, ld - w elements further.
// The squares are summed in float64: the update does not depend on the scale of
// M, and the square of an entry above ~1.8e19 overflows float32.
template <int GDT>
__global__ __launch_bounds__(kMomThreads) void momentum_sumsq_kernel(float* M, const void* G, const ProblemDesc* probs,
                                                                     int64_t per_problem, int64_t chunks, float mu,
                                                                     double* partials) {
  __shared__ double red[kMomThreads / 64];
  const int64_t b = blockIdx.x;
  const int64_t p = b / chunks;
  const int64_t c = b - p * chunks;
  const int64_t first = c * kMomChunk;                      // first element of the block within the problem
  const int len = static_cast<int>(min<int64_t>(kMomChunk, per_problem - first));
  const ProblemDesc pd = probs[p];
  const int tid = threadIdx.x;
  const int e0 = tid * 4;
  // the thread's first element: stored address i0, column c0 of a w-wide row
  // (w = INT_MAX for a contiguous problem: its rows run into each other)
  int64_t i0;
  int c0, w;
  if (pd.ld == pd.w) {
    i0 = pd.src_off + first + e0;
    c0 = 0;
    w = 0x7fffffff;
  } else {
    const int64_t e = first + e0;
    const int64_t r = e / pd.w;
    c0 = static_cast<int>(e - r * pd.w);
    i0 = pd.src_off + r * pd.ld + c0;
    w = pd.w;
  }
  double ss = 0.0;
  // the vector path needs 4 elements in one row and 16-byte aligned momentum
  // (a block's rows need not be: a split block or column block whose width is
  // not a multiple of 4, or a matrix at an offset that is not)
  if (e0 + 4 <= len && c0 + 4 <= w && (i0 & 3) == 0) {
    float g[4];
    load_grad4<GDT>(G, i0, g);
    f32x4* mp = reinterpret_cast<f32x4*>(M + i0);
    f32x4 m = *mp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[e] = mu * m[e] + g[e];
      ss += static_cast<double>(m[e]) * m[e];
    }
    *mp = m;
  } else if (e0 < len) {
    int64_t i = i0;
    int c = c0;
    for (int e = e0; e < min(e0 + 4, len); ++e) {
      const float m = mu * M[i] + grad_to_f32<GDT>(G, i);
      M[i] = m;
      ss += static_cast<double>(m) * m;
      ++i;
      if (++c == w) {   // next row of the block
        c = 0;
        i += pd.ld - w;
      }
    }
  }
  ss = wave_sum_d(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) partials[b] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_momentum_sumsq(int grad_dtype, float* M, const void* G, const ProblemDesc* probs, int n_problems,
                                 int64_t per_problem, int64_t chunks, float mu, double* partials, hipStream_t s) {
  static_assert(kMomThreads == 256, "the block reduction sums four waves");
  const int64_t blocks = static_cast<int64_t>(n_problems) * chunks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (grad_dtype) {
    case MUON_DTYPE_BF16:
      hipLaunchKernelGGL(momentum_sumsq_kernel<MUON_DTYPE_BF16>, dim3(blocks), dim3(kMomThreads), 0, s, M, G, probs,
                         per_problem, chunks, mu, partials);
      break;
    case MUON_DTYPE_F16:
      hipLaunchKernelGGL(momentum_sumsq_kernel<MUON_DTYPE_F16>, dim3(blocks), dim3(kMomThreads), 0, s, M, G, probs,
                         per_problem, chunks, mu, partials);
      break;
    default:
      hipLaunchKernelGGL(momentum_sumsq_kernel<MUON_DTYPE_F32>, dim3(blocks), dim3(kMomThreads), 0, s, M, G, probs,
                         per_problem, chunks, mu, partials);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 1 / (||Y||_F + eps) per problem; partial sums combined in double, fixed order

// One block per problem: thread t sums partials t, t + 256, ... into four
// float64 accumulators (k mod 4), combined in a fixed order, then waves and the
// block in a fixed order; the result depends only on the problem's own partials.
__global__ __launch_bounds__(256) void finalize_norm_kernel(const double* partials, int64_t chunks, float eps,
                                                            float* inv_norm) {
  __shared__ double red[4];
  const int p = blockIdx.x;
  const int tid = threadIdx.x;
  const double* part = partials + static_cast<int64_t>(p) * chunks;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t k = tid;
  for (; k + 3 * 256 < chunks; k += 4 * 256) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += part[k + u * 256];
  }
  for (int u = 0; k < chunks; k += 256, ++u) acc[u] += part[k];
  double s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  s = wave_sum_d(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) inv_norm[p] = static_cast<float>(1.0 / (sqrt((red[0] + red[1]) + (red[2] + red[3])) +
                                                        static_cast<double>(eps)));
}

hipError_t launch_finalize_norm(const double* partials, int64_t chunks, int n_problems, float eps, float* inv_norm,
                                hipStream_t s) {
  if (n_problems <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_norm_kernel, dim3(n_problems), dim3(256), 0, s, partials, chunks, eps, inv_norm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// X0 = round(M / (||M||_F + eps)) in canonical orientation (short side = rows),
// written as X (mp x np, row-major), in 64x64 tiles. A matrix
// stored as is goes straight through; one stored transposed is read in its
// stored orientation (coalesced) and turned in LDS. Padding rows/columns are
// written as zeros.

// 4 consecutive elements, rounded to T from materialised fp32 values
template <typename T>
__device__ __forceinline__ void store4(T* dst, const float (&v)[4]) {
  if constexpr (sizeof(T) == 4) {
    f32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = v[e];
    *reinterpret_cast<f32x4*>(dst) = w;
  } else {
    T r[4];
    rne<T, 4>(v, r);
    u16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(unsigned short, r[e]);
    *reinterpret_cast<u16x4*>(dst) = w;
  }
}

// Every block moves 64 KB of momentum. A matrix stored as is is streamed in row
// pieces: the block covers 16 rows x 1024 columns, wave w rows 4 w .. 4 w + 3, and
// in round q (0..15) lane l reads columns 256 (q % 4) + 4 l .. + 3 of row q / 4 of
// the wave's rows, so every wave instruction reads 1 KB of one row and each row
// piece is 4 KB long. A matrix stored transposed goes through LDS in four 64x64
// tiles down a tile column.

template <typename T>
__global__ __launch_bounds__(256) void prep_x0_kernel(const float* M, const ProblemDesc* probs, const float* inv_norm,
                                                      int m, int n, int mp, int np, T* X) {
  __shared__ float tile[64][65];
  const int tiles_j = np >> 6;
  const int per_t = ((mp + 255) >> 8) * tiles_j;       // blocks of a transposed problem
  const int pieces_j = (np + 1023) >> 10;
  const int per_r = (mp >> 4) * pieces_j;              // blocks of a problem stored as is
  const int per = max(per_t, per_r);
  const int p = blockIdx.x / per;
  const int t = blockIdx.x - p * per;
  const ProblemDesc pd = probs[p];
  const float inv = inv_norm[p];
  T* Xp = X + p * static_cast<int64_t>(mp) * np;

  if (!pd.transposed) {
    // stored m x n: element (i, j) at src + i * ld + j
    if (t >= per_r) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = (t / pieces_j) * 16 + 4 * w, c0 = (t % pieces_j) * 1024 + 4 * lane;
    float v[16][4];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int gi = r0 + (q >> 2), gj = c0 + 256 * (q & 3);
      const int64_t base = pd.src_off + static_cast<int64_t>(gi) * pd.ld + gj;
      if (gi < m && gj + 4 <= n && (base & 3) == 0) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(M + base);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[q][e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[q][e] = (gi < m && gj + e < n) ? M[base + e] : 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int gi = r0 + (q >> 2), gj = c0 + 256 * (q & 3);
      if (gj < np) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[q][e] * inv;
        store4<T>(Xp + static_cast<int64_t>(gi) * np + gj, o);
      }
    }
    return;
  }

  if (t >= per_t) return;
  // stored n x m: element (i, j) at src + j * ld + i. The block covers canonical rows
  // i0 .. i0 + 255 (tiles q = 0..3 of 64 rows) and columns j0 .. j0 + 63: stored rows
  // j0 .. j0 + 63, read in 1 KB pieces. All loads are issued first; each tile is
  // then turned in LDS: stored row j0 + 16 k + rr holds canonical column j, and its
  // elements i0 + 64 q + c4 .. + 3 canonical rows.
  const int i0 = (t / tiles_j) * 256, j0 = (t % tiles_j) * 64;
  const int nt = min(4, (mp - i0) >> 6);   // tiles of this block
  const int rr = threadIdx.x >> 4, c4 = (threadIdx.x & 15) * 4;
  float v[4][4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sj = j0 + 16 * k + rr, si = i0 + 64 * q + c4;
        const int64_t base = pd.src_off + static_cast<int64_t>(sj) * pd.ld + si;
        if (sj < n && si + 4 <= m && (base & 3) == 0) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(M + base);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[q][k][e] = w[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[q][k][e] = (sj < n && si + e < m) ? M[base + e] : 0.0f;
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nt) {
      if (q > 0) __syncthreads();   // the previous tile's reads are done
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[c4 + e][16 * k + rr] = v[q][k][e];
      __syncthreads();   // the transposed flag is the same for the whole block
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 16 * k + rr;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = tile[r][c4 + e] * inv;
        store4<T>(Xp + static_cast<int64_t>(i0 + 64 * q + r) * np + j0 + c4, o);
      }
    }
  }
}

hipError_t launch_prep_x0(int ns_dtype, const float* M, const ProblemDesc* probs, const float* inv_norm,
                          int n_problems, int m, int n, int mp, int np, void* X, hipStream_t s) {
  const int64_t per = std::max<int64_t>(static_cast<int64_t>((mp + 255) / 256) * (np / 64),
                                       static_cast<int64_t>(mp / 16) * ((np + 1023) / 1024));
  const int64_t blocks = static_cast<int64_t>(n_problems) * per;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (ns_dtype) {
    case MUON_DTYPE_BF16:
      hipLaunchKernelGGL(prep_x0_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, M, probs, inv_norm, m, n, mp, np,
                         static_cast<__bf16*>(X));
      break;
    case MUON_DTYPE_F16:
      hipLaunchKernelGGL(prep_x0_kernel<_Float16>, dim3(blocks), dim3(256), 0, s, M, probs, inv_norm, m, n, mp, np,
                         static_cast<_Float16*>(X));
      break;
    default:
      hipLaunchKernelGGL(prep_x0_kernel<float>, dim3(blocks), dim3(256), 0, s, M, probs, inv_norm, m, n, mp, np,
                         static_cast<float*>(X));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// AdamW (the article's Adam fallback for non-2D parameters, AdamW mode)

// Two elements per thread, one pass, no loop: with four buffers read and three
// written per element, small per-thread work keeps the most requests in flight.
template <int GDT>
__global__ __launch_bounds__(256) void adamw_kernel(float* p, const void* g, float* m, float* v, int64_t n, float b1,
                                                    float b2, float step_size, float inv_bc2, float eps, float decay) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 2;
  if (i >= n) return;
  auto one = [&](float gi, float& pi, float& mi, float& vi) {
    const float mn = b1 * mi + (1.0f - b1) * gi;
    const float vn = b2 * vi + (1.0f - b2) * gi * gi;
    mi = mn;
    vi = vn;
    pi = pi * decay - step_size * (mn / (sqrtf(vn * inv_bc2) + eps));
  };
  if (i + 2 <= n) {
    float gg[2];
    load_grad2<GDT>(g, i, gg);
    f32x2* pp = reinterpret_cast<f32x2*>(p + i);
    f32x2* mp = reinterpret_cast<f32x2*>(m + i);
    f32x2* vp = reinterpret_cast<f32x2*>(v + i);
    // every byte is touched once per step: non-temporal accesses keep the
    // stream from displacing cached data (about 10% faster than plain ones)
    f32x2 P = __builtin_nontemporal_load(pp), Mv = __builtin_nontemporal_load(mp), Vv = __builtin_nontemporal_load(vp);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float pe = P[e], me = Mv[e], ve = Vv[e];
      one(gg[e], pe, me, ve);
      P[e] = pe; Mv[e] = me; Vv[e] = ve;
    }
    __builtin_nontemporal_store(P, pp);
    __builtin_nontemporal_store(Mv, mp);
    __builtin_nontemporal_store(Vv, vp);
  } else {
    one(grad_to_f32<GDT>(g, i), p[i], m[i], v[i]);
  }
}

hipError_t launch_adamw(int grad_dtype, float* p, const void* g, float* m, float* v, int64_t n, float beta1,
                        float beta2, float step_size, float inv_bc2, float eps, float decay, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 511) / 512;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (grad_dtype) {
    case MUON_DTYPE_BF16:
      hipLaunchKernelGGL(adamw_kernel<MUON_DTYPE_BF16>, dim3(blocks), dim3(256), 0, s, p, g, m, v, n, beta1, beta2,
                         step_size, inv_bc2, eps, decay);
      break;
    case MUON_DTYPE_F16:
      hipLaunchKernelGGL(adamw_kernel<MUON_DTYPE_F16>, dim3(blocks), dim3(256), 0, s, p, g, m, v, n, beta1, beta2,
                         step_size, inv_bc2, eps, decay);
      break;
    default:
      hipLaunchKernelGGL(adamw_kernel<MUON_DTYPE_F32>, dim3(blocks), dim3(256), 0, s, p, g, m, v, n, beta1, beta2,
                         step_size, inv_bc2, eps, decay);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bit-exact batched copies (pack / unpack)

struct CopyBatch {
  CopyItem items[kCopyBatch];
};

__global__ __launch_bounds__(256) void copy_batch_kernel(CopyBatch b) {
  const CopyItem it = b.items[blockIdx.y];
  const char* s = static_cast<const char*>(it.src);
  char* d = static_cast<char*>(it.dst);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  int64_t done = 0;
  if (((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(d)) & 15) == 0) {
    const int64_t nv = it.bytes >> 4;
    const uint4* sv = reinterpret_cast<const uint4*>(s);
    uint4* dv = reinterpret_cast<uint4*>(d);
    for (int64_t k = t0; k < nv; k += stride) dv[k] = sv[k];
    done = nv << 4;
  }
  for (int64_t k = done + t0; k < it.bytes; k += stride) d[k] = s[k];
}

// ---------------------------------------------------------------------------
// zeros over `count` regions of `bytes` bytes, `stride` bytes apart (16-byte
// aligned, bytes a multiple of 16)

__global__ __launch_bounds__(256) void zero_regions_kernel(char* base, int64_t stride, int64_t n16, int64_t count) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t tstride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t p = blockIdx.y; p < count; p += gridDim.y) {
    uint4* d = reinterpret_cast<uint4*>(base + p * stride);
    for (int64_t k = t0; k < n16; k += tstride) d[k] = uint4{0u, 0u, 0u, 0u};
  }
}

hipError_t launch_zero_regions(void* base, int64_t stride, int64_t bytes, int64_t count, hipStream_t s) {
  if (count <= 0 || bytes <= 0) return hipSuccess;
  if (((reinterpret_cast<uintptr_t>(base) | static_cast<uint64_t>(stride) | static_cast<uint64_t>(bytes)) & 15) != 0)
    return hipErrorInvalidValue;
  const int64_t n16 = bytes >> 4;
  const int64_t gx = std::min<int64_t>((n16 + 255) / 256, 64);
  const int64_t gy = std::min<int64_t>(count, 65535);
  hipLaunchKernelGGL(zero_regions_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), dim3(256), 0, s,
                     static_cast<char*>(base), stride, n16, count);
  return hipGetLastError();
}

hipError_t launch_copy_batch(const CopyItem* items, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  CopyBatch b;
  int64_t maxb = 0;
  for (int i = 0; i < n; ++i) {
    b.items[i] = items[i];
    if (items[i].bytes > maxb) maxb = items[i].bytes;
  }
  int64_t gx = (maxb / 16 + 255) / 256;
  if (gx < 1) gx = 1;
  if (gx > 1024) gx = 1024;
  hipLaunchKernelGGL(copy_batch_kernel, dim3(gx, n), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace muon
