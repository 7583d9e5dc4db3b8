// Batched MFMA GEMM of the Newton-Schulz iteration (gfx950).
//
// Every product of the iteration is written in "NT" form, C = P * Q^T, where
// both operands are row-major with the contraction index contiguous:
//   A = X X^T          P = X,  Q = X                 (symmetric output)
//   A A  (A symmetric) P = A,  Q = A                 (symmetric output)
//   B X                P = B,  Q = Y = X^T           (Y is kept alongside X)
//   Gram: R0 = X0 X0^T, R R, R Q, Q (R Q), Q P, P X0 likewise.
// Keeping both X and X^T (the update's epilogue writes both) removes every
// transposed operand load from the main loop.
//
// Tile: TILE x TILE outputs per workgroup (256 or 128), 4 waves in a 2x2 grid,
// each wave owning (TILE/2)^2 outputs as 32x32 MFMA blocks. K advances in
// 128-byte slices (64 bf16/f16 or 32 f32 elements). Operand slices go straight
// from global memory to LDS (global_load_lds_dwordx4) into a double buffer;
// rows are 128 bytes, with the 16-byte chunk index XOR-swizzled by the row so
// that the MFMA operand reads (ds_read_b128, 32 rows at one chunk) spread over
// all banks. One barrier per K slice.
//
// Epilogue: each wave stages 32 rows of its fp32 accumulators in LDS, applies
//   v = alpha * acc + beta * D[i][j] + gamma * [i == j]
// and stores v (rounded to the element type) row-major to C and/or transposed
// to Ct; a symmetric launch computes only tiles with ti >= tj and mirrors them
// (on diagonal tiles each element is written exactly once, so the stored matrix
// is exactly symmetric). The apply epilogue instead finishes the Muon step,
// p <- p * decay - lr * v, at the matrix's stored (possibly transposed) position.
#include "common.hpp"
#include "kernels.hpp"

namespace muon {

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  using V = bf16x8;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  using V = f16x8;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  using V = f32x4;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    // a 16-byte chunk holds 4 consecutive k; lanes 0-31 and 32-63 hold adjacent chunks
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  }
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so that neighbours share its L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, k = b >> 3;
  return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { using U = u16x8; };
template <> struct Vec8<_Float16> { using U = u16x8; };

// load 8 consecutive elements of type T as floats (16-byte aligned for 16-bit T)
template <typename T> __device__ __forceinline__ void ld8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  } else {
    u16x8 u = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(__builtin_bit_cast(T, (unsigned short)u[e]));
  }
}

template <typename T> __device__ __forceinline__ void st8(T* p, const T (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[e + 4]; }
    f32x4* q = reinterpret_cast<f32x4*>(p);
    q[0] = a; q[1] = b;
  } else {
    u16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = __builtin_bit_cast(unsigned short, v[e]);
    *reinterpret_cast<u16x8*>(p) = u;
  }
}

template <typename T, int TILE, bool SYM, int EPI>
__global__ __launch_bounds__(256) void ns_gemm(GemmArgs a) {
  constexpr int ESZ = sizeof(T);
  constexpr int HALF = TILE / 2;          // wave tile edge
  constexpr int WB = HALF / 32;           // 32x32 blocks per wave edge
  constexpr int OPB = TILE * 128;         // bytes of one operand slice
  constexpr int LOADS = TILE / 32;        // 1-KB direct loads per wave per operand
  constexpr int SP = HALF + 4;            // staging row pitch (floats)
  using V = typename Mfma<T>::V;

  __shared__ __attribute__((aligned(1024))) char lds0[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * OPB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile decode
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int prob = bid / a.tiles_per_problem;
  const int t = bid - prob * a.tiles_per_problem;
  int ti, tj;
  if constexpr (SYM) {
    ti = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    tj = t - ti * (ti + 1) / 2;
  } else {
    constexpr int G = 4;
    const int per_group = G * a.tiles_n;
    const int g = t / per_group;
    const int first = g * G;
    const int gsz = min(a.tiles_m - first, G);
    const int w = t - g * per_group;
    ti = first + w % gsz;
    tj = w / gsz;
  }

  // ---- per-lane direct-load offsets (bytes, relative to the tile's first row)
  const char* Pb = static_cast<const char*>(a.P) +
                   (static_cast<int64_t>(prob) * a.p_ps + static_cast<int64_t>(ti) * TILE * a.ldp) * ESZ;
  const char* Qb = static_cast<const char*>(a.Q) +
                   (static_cast<int64_t>(prob) * a.q_ps + static_cast<int64_t>(tj) * TILE * a.ldq) * ESZ;
  int64_t poff[LOADS], qoff[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int r = (wave * LOADS + it) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    poff[it] = static_cast<int64_t>(r) * a.ldp * ESZ + c * 16;
    qoff[it] = static_cast<int64_t>(r) * a.ldq * ESZ + c * 16;
  }

  auto issue = [&](char* st, int kt) {
    const int64_t kb = static_cast<int64_t>(kt) * 128;
#pragma unroll
    for (int it = 0; it < LOADS; ++it)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Pb + poff[it] + kb),
                                       (MUON_LDS void*)(st + (wave * LOADS + it) * 1024), 16, 0, 0);
#pragma unroll
    for (int it = 0; it < LOADS; ++it)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Qb + qoff[it] + kb),
                                       (MUON_LDS void*)(st + OPB + (wave * LOADS + it) * 1024), 16, 0, 0);
  };

  // ---- per-lane MFMA operand read offsets (bytes within an operand slice)
  int aoff[WB][4], boff[WB][4];
#pragma unroll
  for (int i = 0; i < WB; ++i) {
    const int ra = wm * HALF + i * 32 + (lane & 31);
    const int rb = wn * HALF + i * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      aoff[i][ks] = ra * 128 + ((c ^ swz(ra)) << 4);
      boff[i][ks] = rb * 128 + ((c ^ swz(rb)) << 4);
    }
  }

  f32x16 acc[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = a.K / (128 / ESZ);
  issue(lds0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = (kt & 1) ? lds1 : lds0;
    char* nxt = (kt & 1) ? lds0 : lds1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(nxt, kt + 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      V af[WB], bf[WB];
#pragma unroll
      for (int i = 0; i < WB; ++i) af[i] = *reinterpret_cast<const V*>(cur + aoff[i][ks]);
#pragma unroll
      for (int j = 0; j < WB; ++j) bf[j] = *reinterpret_cast<const V*>(cur + OPB + boff[j][ks]);
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) Mfma<T>::run(af[i], bf[j], acc[i][j]);
    }
  }

  // ---- epilogue
  float* stg = reinterpret_cast<float*>((wave < 2 ? lds0 : lds1) + (wave & 1) * 32 * SP * 4);
  const int gi_w = ti * TILE + wm * HALF;   // first row of this wave's outputs
  const int gj_w = tj * TILE + wn * HALF;   // first column
  const bool diag = SYM && (ti == tj);

  int transposed = 0;
  int64_t src = 0;
  if constexpr (EPI == EPI_APPLY) {
    const ProblemDesc pd = a.probs[prob];
    transposed = pd.transposed;
    src = pd.src_off;
  }

  T* C = static_cast<T*>(a.C);
  T* Ct = static_cast<T*>(a.Ct);
  const T* D = static_cast<const T*>(a.D);
  const bool need_col = (EPI == EPI_APPLY) ? (transposed != 0) : (Ct != nullptr);

#pragma unroll
  for (int i = 0; i < WB; ++i) {
    __syncthreads();   // every wave is past its last LDS read (main loop or previous block)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stg[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * SP + j * 32 + (lane & 31)] = acc[i][j][r];
    __syncthreads();

    // row pass: 8 consecutive columns per task
    constexpr int CPR = HALF / 8;            // chunks per row
#pragma unroll 2
    for (int q = lane; q < 32 * CPR; q += 64) {
      const int rr = q / CPR;
      const int cc = (q - rr * CPR) * 8;
      const int gi = gi_w + i * 32 + rr;
      const int gj = gj_w + cc;
      float v[8];
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(stg + rr * SP + cc);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(stg + rr * SP + cc + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = a.alpha * s0[e]; v[e + 4] = a.alpha * s1[e]; }
      if (D != nullptr) {
        float d[8];
        ld8<T>(D + static_cast<int64_t>(prob) * a.d_ps + static_cast<int64_t>(gi) * a.ldd + gj, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += a.beta * d[e];
      }
      if (a.gamma != 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gi == gj + e) v[e] += a.gamma;
      }
      if constexpr (EPI == EPI_APPLY) {
        if (!transposed) {
          const int m = a.m_valid, n = a.n_valid;
          if (gi < m && gj < n) {
            const int64_t idx = src + static_cast<int64_t>(gi) * n + gj;
            if (gj + 8 <= n && (idx & 7) == 0) {
              f32x4* pp = reinterpret_cast<f32x4*>(a.params + idx);
              f32x4 p0 = pp[0], p1 = pp[1];
              f32x4 o0, o1;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                o0[e] = p0[e] * a.decay - a.lr * v[e];
                o1[e] = p1[e] * a.decay - a.lr * v[e + 4];
              }
              pp[0] = o0; pp[1] = o1;
              if (a.update_out) {
                f32x4 u0, u1;
#pragma unroll
                for (int e = 0; e < 4; ++e) { u0[e] = v[e]; u1[e] = v[e + 4]; }
                f32x4* up = reinterpret_cast<f32x4*>(a.update_out + idx);
                up[0] = u0; up[1] = u1;
              }
              if (a.shadow) {
                u16x8 sh;
#pragma unroll
                for (int e = 0; e < 4; ++e) { sh[e] = bf16_bits(o0[e]); sh[e + 4] = bf16_bits(o1[e]); }
                *reinterpret_cast<u16x8*>(a.shadow + idx) = sh;
              }
            } else {
              for (int e = 0; e < 8 && gj + e < n; ++e) {
                const float pn = a.params[idx + e] * a.decay - a.lr * v[e];
                a.params[idx + e] = pn;
                if (a.update_out) a.update_out[idx + e] = v[e];
                if (a.shadow) a.shadow[idx + e] = bf16_bits(pn);
              }
            }
          }
        } else {
          float4* sp = reinterpret_cast<float4*>(stg + rr * SP + cc);
          sp[0] = make_float4(v[0], v[1], v[2], v[3]);
          sp[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
      } else {
        T o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e]);
        if (C != nullptr) {
          T* cp = C + static_cast<int64_t>(prob) * a.c_ps + static_cast<int64_t>(gi) * a.ldc + gj;
          if (!diag || gi >= gj + 7) {
            st8<T>(cp, o);
          } else {
            for (int e = 0; e < 8; ++e)
              if (gi >= gj + e) cp[e] = o[e];
          }
        }
        if (need_col) {
          float4* sp = reinterpret_cast<float4*>(stg + rr * SP + cc);
          sp[0] = make_float4(to_f32(o[0]), to_f32(o[1]), to_f32(o[2]), to_f32(o[3]));
          sp[1] = make_float4(to_f32(o[4]), to_f32(o[5]), to_f32(o[6]), to_f32(o[7]));
        }
      }
    }

    if (need_col) {
      __syncthreads();
      // column pass: 8 consecutive rows of one column per task
#pragma unroll 2
      for (int q = lane; q < HALF * 4; q += 64) {
        const int r8 = (q & 3) * 8;
        const int cc = q >> 2;
        const int gi = gi_w + i * 32 + r8;
        const int gj = gj_w + cc;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stg[(r8 + e) * SP + cc];
        if constexpr (EPI == EPI_APPLY) {
          // stored n x m (rows > cols): element (gi, gj) of the canonical matrix is at gj * m + gi
          const int m = a.m_valid, n = a.n_valid;
          if (gj < n && gi < m) {
            const int64_t idx = src + static_cast<int64_t>(gj) * m + gi;
            if (gi + 8 <= m && (idx & 7) == 0) {
              f32x4* pp = reinterpret_cast<f32x4*>(a.params + idx);
              f32x4 p0 = pp[0], p1 = pp[1];
              f32x4 o0, o1;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                o0[e] = p0[e] * a.decay - a.lr * v[e];
                o1[e] = p1[e] * a.decay - a.lr * v[e + 4];
              }
              pp[0] = o0; pp[1] = o1;
              if (a.update_out) {
                f32x4 u0, u1;
#pragma unroll
                for (int e = 0; e < 4; ++e) { u0[e] = v[e]; u1[e] = v[e + 4]; }
                f32x4* up = reinterpret_cast<f32x4*>(a.update_out + idx);
                up[0] = u0; up[1] = u1;
              }
              if (a.shadow) {
                u16x8 sh;
#pragma unroll
                for (int e = 0; e < 4; ++e) { sh[e] = bf16_bits(o0[e]); sh[e + 4] = bf16_bits(o1[e]); }
                *reinterpret_cast<u16x8*>(a.shadow + idx) = sh;
              }
            } else {
              for (int e = 0; e < 8 && gi + e < m; ++e) {
                const float pn = a.params[idx + e] * a.decay - a.lr * v[e];
                a.params[idx + e] = pn;
                if (a.update_out) a.update_out[idx + e] = v[e];
                if (a.shadow) a.shadow[idx + e] = bf16_bits(pn);
              }
            }
          }
        } else {
          T o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e]);
          T* cp = Ct + static_cast<int64_t>(prob) * a.ct_ps + static_cast<int64_t>(gj) * a.ldct + gi;
          if (!diag || gi > gj) {
            st8<T>(cp, o);
          } else {
            for (int e = 0; e < 8; ++e)
              if (gi + e > gj) cp[e] = o[e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers

template <typename T, int TILE, bool SYM, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  if (a.total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((ns_gemm<T, TILE, SYM, EPI>), dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int TILE>
static hipError_t launch_tile(bool sym, int epi, const GemmArgs& a, hipStream_t s) {
  if (epi == EPI_APPLY) return launch_t<T, TILE, false, EPI_APPLY>(a, s);
  return sym ? launch_t<T, TILE, true, EPI_STORE>(a, s) : launch_t<T, TILE, false, EPI_STORE>(a, s);
}

template <typename T>
static hipError_t launch_dtype(int tile, bool sym, int epi, const GemmArgs& a, hipStream_t s) {
  return tile == 256 ? launch_tile<T, 256>(sym, epi, a, s) : launch_tile<T, 128>(sym, epi, a, s);
}

hipError_t launch_ns_gemm(int dtype, int tile, bool sym, int epi, const GemmArgs& a, hipStream_t s) {
  switch (dtype) {
    case MUON_DTYPE_BF16: return launch_dtype<__bf16>(tile, sym, epi, a, s);
    case MUON_DTYPE_F16: return launch_dtype<_Float16>(tile, sym, epi, a, s);
    default: return launch_dtype<float>(tile, sym, epi, a, s);
  }
}

}  // namespace muon
