// Batched MFMA GEMM of the Newton-Schulz iteration (gfx950).
//
// The first operand P is always row-major with the contraction index K
// contiguous. The second operand comes in two layouts:
//   NT (symmetric launches): Q is N x K, K contiguous, C = P Q^T
//     A = X X^T          P = X,  Q = X
//     A A  (A symmetric) P = A,  Q = A
//     Gram: R0 = X0 X0^T, Q = a I + b R + c R R, T = R Q, R <- Q T (Q and T
//     are stored symmetric, so they serve as their own transposes)
//   NN (full launches): Q is K x N, N contiguous, C = P Q
//     B X                P = B,  Q = X
//     Gram: Q P, P X0
// The NN operand is staged in LDS as K rows and read with the transposed LDS
// read of gfx950, so X is stored only once, row-major, and no product needs a
// transposed copy of its operand.
//
// Tile: TILE x TILE outputs per workgroup (256 or 128), 4 waves in a 2x2 grid,
// each wave owning (TILE/2)^2 outputs as 32x32 MFMA blocks. K advances in
// 128-byte slices (64 bf16/f16 or 32 f32 elements). Operand slices are staged
// through registers into a double buffer in LDS. K-contiguous operands use
// 128-byte rows, with the 16-byte chunk index XOR-swizzled by the row so that
// the MFMA operand reads (ds_read_b128, 32 rows at one chunk) spread over all
// banks; an NN operand uses rows of TILE elements with the 32-byte pair index
// XOR-swizzled by the row, so the four rows of a transposed read fall in
// different banks. MFMA operands are double-buffered in registers so that reads of
// the next sub-step overlap the current MFMAs; one barrier per K slice.
//
// Epilogue: each wave stages 32 rows of its fp32 accumulators in LDS, applies
//   v = alpha * acc + beta * D[i][j] + gamma * [i == j]
// and stores v (rounded to the element type) row-major to C and/or transposed
// to Ct; a symmetric launch computes only tiles with ti >= tj and mirrors them
// (on diagonal tiles each element is written exactly once, so the stored matrix
// is exactly symmetric). The apply epilogue instead finishes the Muon step,
// p <- p * decay - lr * v (fp32 or bf16 params), at the matrix's stored (possibly
// transposed) position, for the elements of the problem's window (the whole
// problem in an ordinary step).
// Global loads of the epilogue (D, params) are issued in batches ahead of use.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace muon {

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  using V = bf16x8;
  static constexpr int kInstr = 1;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  using V = f16x8;
  static constexpr int kInstr = 1;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  using V = f32x4;
  static constexpr int kInstr = 4;
  static __device__ __forceinline__ void run(const V& a, const V& b, f32x16& c) {
    // a 16-byte chunk holds 4 consecutive k; lanes 0-31 and 32-63 hold adjacent chunks
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  }
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Products are issued with the K x N operand first, so a 32 x 32 accumulator
// block holds the transposed tile block: register 4 q + e of lane l is row l % 32,
// column 8 q + 4 (l / 32) + e. Four consecutive columns of one row go to the
// epilogue staging area in one 16-byte write.
__device__ __forceinline__ void stage4(float* dst, const f32x16& acc, int q) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
}

// Pair swizzle of the K x N operand (rows of 32-byte pairs in LDS): pair p of K row
// kr is stored at pair slot p ^ nn_swz(kr). A 16-bit transposed read takes, per
// half wave, two adjacent pairs (2q, 2q + 1) from four consecutive K rows; the
// slots of those rows differ in bits 1-2, so the eight 32-byte reads fall in eight
// different bank groups. An fp32 read takes four pairs from rows kr and kr + 4,
// whose slots differ in bit 2. Row writes stay a permutation of each row.
__device__ __forceinline__ int nn_swz(int kr) { return ((kr & 3) << 1) ^ (kr & 4); }

// Transposed LDS read of 16-bit elements (gfx950 ds_read_b64_tr_b16). In each
// group of 16 lanes, lane s supplies the address of 4 consecutive elements;
// lane l of the group receives element l % 4 of the rows addressed by lanes
// l / 4, l / 4 + 4, l / 4 + 8 and l / 4 + 12. With lane s pointing at row
// s / 4, columns 4 (s % 4) .. + 3 of a 4 x 16 block, lane l receives column l of
// the block, rows 0..3: one MFMA operand quarter read across rows.
template <typename T> struct TrRead;
template <> struct TrRead<__bf16> {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4;
  static __device__ __forceinline__ v4 get(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) v4*)(p));
  }
};
template <> struct TrRead<_Float16> {
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 v4;
  static __device__ __forceinline__ v4 get(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) v4*)(p));
  }
};

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

// Tile geometry shared by the main loops and the epilogue.
template <typename T, int TILE> struct Geo {
  static constexpr int ESZ = sizeof(T);
  static constexpr int HALF = TILE / 2;          // wave tile edge (2 x 2 waves)
  static constexpr int WB = HALF / 32;           // 32x32 blocks per wave edge
  static constexpr int OPB = TILE * 128;         // bytes of one operand slice
  static constexpr int LOADS = TILE / 32;        // 1-KB direct loads per wave per operand
  static constexpr int SP = HALF + 4;            // staging row pitch (floats)
  using V = typename Mfma<T>::V;
};

// Logical tile (problem, tile row, tile column) of block b of a launch.
// Both kinds of launch cut each problem into bands of kBand tile columns (the
// last band may be narrower). Full launches walk a band row by row. Symmetric
// launches (lower tiles only) walk a band from its diagonal down: first the
// small triangle of rows whose band columns reach the diagonal, then full rows
// of kBand tiles. Workgroups are dealt round-robin over the 8 XCDs, so with 16
// tile rows XCD x runs tiles of 8 tile rows and one column per band: per XCD and
// per problem, 8 row strips of P and 4 column strips of Q meet in its
// last-level cache, where a column-major walk spreads 2 row strips over all 16
// columns (12 strips against 18). Against column-major walks: 1.5% faster on
// 4096-row updates, 1-3.5% on X X^T launches.
constexpr int kBand = 4;

template <bool SYM>
__device__ __forceinline__ void decode_tile(const GemmArgs& a, int b, int& prob, int& ti, int& tj) {
  prob = b / a.tiles_per_problem;
  int t = b - prob * a.tiles_per_problem;
  if constexpr (SYM) {
    const int T = a.tiles_m;
    int c0 = 0, w = min(kBand, T);
    // a band of width w starting at column c0 holds w (w + 1) / 2 + w (T - c0 - w) tiles
    for (int nb = w * (w + 1) / 2 + w * (T - w); t >= nb; nb = w * (w + 1) / 2 + w * (T - c0 - w)) {
      t -= nb;
      c0 += kBand;
      w = min(kBand, T - c0);
    }
    const int tri = w * (w + 1) / 2;
    if (t < tri) {              // rows c0 .. c0 + w - 1 hold 1, 2, .. w tiles
      int r = 0;
      while (t > r) {
        t -= r + 1;
        ++r;
      }
      ti = c0 + r;
      tj = c0 + t;
    } else {
      t -= tri;
      ti = c0 + w + t / w;
      tj = c0 + t % w;
    }
  } else {
    const int per = kBand * a.tiles_m;
    const int band = t / per;
    const int w = t - band * per;
    const int first = band * kBand;
    const int width = min(a.tiles_n - first, kBand);
    tj = first + w % width;
    ti = w / width;
  }
}

// Main loop: acc[i][j] += P[tile rows] Q[tile cols]^T over the whole K range.
//
// K advances in 128-byte slices through two LDS buffers. Each slice has four
// sub-steps (one per 16-byte chunk pair); the MFMA operands of sub-step s + 1
// are read from LDS while the MFMAs of sub-step s run (two register sets), and
// every sub-step is its own scheduling region, so no MFMA waits for a read
// issued in its own region.
//
// Operand slices are staged through registers: during slice kt, sub-steps 0..2
// each write a third of slice kt + 1 (loaded into registers during slice kt - 1)
// into the other LDS buffer and immediately reload those registers with the same
// part of slice kt + 2. Spreading the global loads over the slice keeps the load
// path busy steadily; issued in one burst per slice (as direct-to-LDS loads must
// be, once the barrier frees their buffer) they stalled the MFMAs for about a
// sixth of the time. Each register waits only for its own load (vmcnt counts
// loads in issue order), so a load has a whole slice of latency to hide. One
// barrier per slice, before the last sub-step, publishes slice kt + 1. The last
// slices reload slice nk - 1 (in bounds, never used).
template <typename T, int TILE, bool NN>
__device__ __forceinline__ void mainloop(const GemmArgs& a, int prob, int ti, int tj, char* lds0, char* lds1,
                                         f32x16 (&acc)[Geo<T, TILE>::WB][Geo<T, TILE>::WB]) {
  using Gm = Geo<T, TILE>;
  constexpr int ESZ = Gm::ESZ, HALF = Gm::HALF, WB = Gm::WB, OPB = Gm::OPB, LOADS = Gm::LOADS;
  constexpr int NV = 2 * LOADS;                       // 16-byte vectors per lane per slice (P, then Q)
  constexpr int NMF = WB * WB * Mfma<T>::kInstr;      // MFMA instructions per sub-step
  constexpr int KS = 128 / ESZ;                       // K elements per slice
  constexpr int RB = TILE * ESZ;                      // NN: bytes of one K row of the Q slice
  constexpr int CPRQ = RB / 16;                       // NN: 16-byte chunks per K row
  // LDS reads per sub-step: A, then B (NN: two transposed quarter reads per 16-bit
  // operand, four element reads per fp32 operand)
  constexpr int BRD = !NN ? 1 : (ESZ == 2 ? 2 : 4);
  constexpr int NRD = WB + WB * BRD;
  using V = typename Gm::V;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-lane global source and LDS destination of each 16-byte vector.
  // P (and Q unless NN): lane l of load `it` covers row (wave * LOADS + it) * 8 +
  // l / 8, chunk l % 8 of a 128-byte K slice; the chunk is stored at position
  // chunk ^ swz(row) of its 128-byte LDS row.
  // NN Q (stored K x N, N contiguous): the slice is KS rows of TILE columns; load
  // `it` of thread t covers chunk (it * 256 + t) of the row-major slice, stored in
  // an RB-byte LDS row with its 32-byte pair index XORed with nn_swz(row).
  const char* Pb = static_cast<const char*>(a.P) +
                   (static_cast<int64_t>(prob) * a.p_ps + static_cast<int64_t>(ti) * TILE * a.ldp) * ESZ;
  const char* Qb = static_cast<const char*>(a.Q) +
                   (static_cast<int64_t>(prob) * a.q_ps +
                    (NN ? static_cast<int64_t>(tj) * TILE : static_cast<int64_t>(tj) * TILE * a.ldq)) * ESZ;
  const char* gp[NV];
  int wofs[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int it = v % LOADS;
    if (NN && v >= LOADS) {
      const int id = it * 256 + static_cast<int>(threadIdx.x);
      const int kr = id / CPRQ, c = id % CPRQ;
      gp[v] = Qb + static_cast<int64_t>(kr) * a.ldq * ESZ + c * 16;
      wofs[v] = OPB + kr * RB + (((c >> 1) ^ nn_swz(kr)) << 5) + ((c & 1) << 4);
    } else {
      const int r = (wave * LOADS + it) * 8 + (lane >> 3);
      const int c = lane & 7;
      if (v < LOADS) gp[v] = Pb + static_cast<int64_t>(r) * a.ldp * ESZ + c * 16;
      else gp[v] = Qb + static_cast<int64_t>(r) * a.ldq * ESZ + c * 16;
      wofs[v] = (v < LOADS ? 0 : OPB) + r * 128 + ((c ^ swz(r)) << 4);
    }
  }
  // byte step of one K slice: 128 bytes along a row, or KS rows of Q for NN
  const int64_t qstep = NN ? static_cast<int64_t>(KS) * a.ldq * ESZ : 128;
  u16x8 rv[NV];
  auto gload = [&](int v0, int v1, int kt) {
    const int64_t kp = static_cast<int64_t>(kt) * 128, kq = static_cast<int64_t>(kt) * qstep;
#pragma unroll
    for (int v = v0; v < v1; ++v) rv[v] = *reinterpret_cast<const u16x8*>(gp[v] + (v < LOADS ? kp : kq));
  };
  auto lwrite = [&](int v0, int v1, char* st) {
#pragma unroll
    for (int v = v0; v < v1; ++v) *reinterpret_cast<u16x8*>(st + wofs[v]) = rv[v];
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
  // NN B operand, offsets at sub-step 0 (sub-step ks adds ks * (KS / 4) rows).
  // 16-bit: lane l (group g = l / 16, s = l % 16) reads quarter h from row
  // 8 (g / 2) + 4 h + s / 4, columns 16 (g % 2) + 4 (s % 4) .. + 3 of block j.
  // fp32: element e of lane l is row 4 (l / 32) + e, column l % 32 of block j.
  int bnn[WB][BRD];
  if constexpr (NN) {
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      const int nb = wn * HALF + j * 32;
#pragma unroll
      for (int h = 0; h < BRD; ++h) {
        int kr, col;
        if constexpr (ESZ == 2) {
          const int g = lane >> 4, sl = lane & 15;
          kr = 8 * (g >> 1) + 4 * h + (sl >> 2);
          col = nb + 16 * (g & 1) + 4 * (sl & 3);
        } else {
          kr = 4 * (lane >> 5) + h;
          col = nb + (lane & 31);
        }
        const int cb = col * ESZ;   // byte column
        bnn[j][h] = OPB + kr * RB + ((((cb >> 5) ^ nn_swz(kr))) << 5) + (cb & 31);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  V fa0[WB], fb0[WB], fa1[WB], fb1[WB];
  auto rd = [&](V (&xa)[WB], V (&xb)[WB], const char* buf, int ks) {
#pragma unroll
    for (int i = 0; i < WB; ++i) xa[i] = *reinterpret_cast<const V*>(buf + aoff[i][ks]);
    if constexpr (!NN) {
#pragma unroll
      for (int j = 0; j < WB; ++j) xb[j] = *reinterpret_cast<const V*>(buf + OPB + boff[j][ks]);
    } else if constexpr (ESZ == 2) {
      const int kofs = ks * (KS / 4) * RB;
#pragma unroll
      for (int j = 0; j < WB; ++j) {
        const auto lo = TrRead<T>::get(buf + bnn[j][0] + kofs);
        const auto hi = TrRead<T>::get(buf + bnn[j][1] + kofs);
        xb[j] = __builtin_bit_cast(V, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
      const int kofs = ks * (KS / 4) * RB;
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) xb[j][e] = *reinterpret_cast<const float*>(buf + bnn[j][e] + kofs);
    }
  };
  auto mm = [&](V (&xa)[WB], V (&xb)[WB]) {
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j) Mfma<T>::run(xb[j], xa[i], acc[i][j]);   // transposed block, see epilogue
  };
  // scheduling of one sub-step: its nw LDS writes and global loads, then its NRD
  // operand reads, each paired with MFMAs; then a fence
  auto region = [&](int nw) {
#pragma unroll
    for (int q = 0; q < nw; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // LDS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // global load
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    }
#pragma unroll
    for (int q = 0; q < NRD; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 1 ? NMF / NRD - 1 : 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = a.K / (128 / ESZ);                   // even: K is a multiple of two slices
  constexpr int B1 = (NV + 2) / 3, B2 = (2 * NV + 2) / 3;
  auto slice = [&](char* cur, char* nxt, int kt) {
    const int kl = min(kt + 2, nk - 1);
    // no explicit vmcnt wait: the compiler waits for each register's own load
    // right before its LDS write, so every load has a whole slice to arrive
    lwrite(0, B1, nxt);
    gload(0, B1, kl);
    rd(fa1, fb1, cur, 1);
    mm(fa0, fb0);
    region(B1);
    lwrite(B1, B2, nxt);
    gload(B1, B2, kl);
    rd(fa0, fb0, cur, 2);
    mm(fa1, fb1);
    region(B2 - B1);
    lwrite(B2, NV, nxt);
    gload(B2, NV, kl);
    rd(fa1, fb1, cur, 3);
    mm(fa0, fb0);
    region(NV - B2);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own LDS writes and reads done
    __syncthreads();
    rd(fa0, fb0, nxt, 0);
    mm(fa1, fb1);
    region(0);
  };

  gload(0, NV, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lwrite(0, NV, lds0);
  gload(0, NV, 1);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  rd(fa0, fb0, lds0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    slice(lds0, lds1, kt);
    slice(lds1, lds0, kt + 1);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

// 8 consecutive elements of T held raw in registers (one or two 16-byte vectors).
template <typename T> struct Pack8 {
  u16x8 u;
  __device__ __forceinline__ void load(const T* p) { u = *reinterpret_cast<const u16x8*>(p); }
  __device__ __forceinline__ float get(int e) const {
    return static_cast<float>(__builtin_bit_cast(T, static_cast<unsigned short>(u[e])));
  }
};
template <> struct Pack8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    lo = q[0];
    hi = q[1];
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

// Parameter access of the apply epilogues: fp32 (EPI_APPLY) or bf16 words
// (EPI_APPLY_BF16), as floats. The 8-element forms need pidx a multiple of 8.
// ParamPack holds 8 parameters as loaded; they are converted where used, so a
// load can stay in flight until then.
template <int EPI> struct ParamPackT { using type = Pack8<float>; };
template <> struct ParamPackT<EPI_APPLY_BF16> { using type = Pack8<__bf16>; };
template <int EPI> using ParamPack = typename ParamPackT<EPI>::type;

template <int EPI>
__device__ __forceinline__ void store_p8(void* params, int64_t pidx, const f32x4& o0, const f32x4& o1) {
  if constexpr (EPI == EPI_APPLY_BF16) {
    u16x8 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) { w[e] = bf16_bits(keep_f32(o0[e])); w[e + 4] = bf16_bits(keep_f32(o1[e])); }
    *reinterpret_cast<u16x8*>(static_cast<unsigned short*>(params) + pidx) = w;
  } else {
    f32x4* pp = reinterpret_cast<f32x4*>(static_cast<float*>(params) + pidx);
    pp[0] = o0;
    pp[1] = o1;
  }
}

template <int EPI>
__device__ __forceinline__ float load_p1(const void* params, int64_t i) {
  if constexpr (EPI == EPI_APPLY_BF16) return bf16_bits_to_f32(static_cast<const unsigned short*>(params)[i]);
  else return static_cast<const float*>(params)[i];
}

template <int EPI>
__device__ __forceinline__ void store_p1(void* params, int64_t i, float v) {
  if constexpr (EPI == EPI_APPLY_BF16) static_cast<unsigned short*>(params)[i] = bf16_bits(keep_f32(v));
  else static_cast<float*>(params)[i] = v;
}

// The launch's apply scalars, read once per workgroup.
struct ApplyScalars {
  void* params;
  float* update_out;
  unsigned short* shadow;
  float decay, lr;
};

// One run of up to 8 consecutive stored elements e0 .. e0 + cnt - 1 of a problem:
// v goes to update_out at uidx (every element), and p <- p * decay - lr * v, with
// the optional bf16 copy of the new p (shadow, fp32 params only), to the params
// at pidx for the elements inside the problem's window [lo, hi). `vec`: a whole
// run inside the window with pidx a multiple of 8 and uidx of 4, whose params
// the caller has loaded into pp; anything else takes the scalar path.
template <int EPI>
__device__ __forceinline__ void apply8(const ApplyScalars& a, int64_t pidx, int64_t uidx, int64_t e0, int cnt,
                                       int64_t lo, int64_t hi, const float (&v)[8], const ParamPack<EPI>& pp,
                                       bool vec) {
  if (vec) {
    f32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = pp.get(e) * a.decay - a.lr * v[e];
      o1[e] = pp.get(e + 4) * a.decay - a.lr * v[e + 4];
    }
    store_p8<EPI>(a.params, pidx, o0, o1);
    if (a.update_out) {
      f32x4 u0, u1;
#pragma unroll
      for (int e = 0; e < 4; ++e) { u0[e] = v[e]; u1[e] = v[e + 4]; }
      f32x4* up = reinterpret_cast<f32x4*>(a.update_out + uidx);
      up[0] = u0;
      up[1] = u1;
    }
    if constexpr (EPI == EPI_APPLY) {
      if (a.shadow) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = o0[e]; x[e + 4] = o1[e]; }
        __bf16 r[8];
        rne<__bf16, 8>(x, r);
        u16x8 sh;
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[e] = __builtin_bit_cast(unsigned short, r[e]);
        *reinterpret_cast<u16x8*>(a.shadow + pidx) = sh;
      }
    }
  } else {
    for (int e = 0; e < cnt; ++e) {
      if (a.update_out) a.update_out[uidx + e] = v[e];
      if (e0 + e >= lo && e0 + e < hi) {
        const float pn = load_p1<EPI>(a.params, pidx + e) * a.decay - a.lr * v[e];
        store_p1<EPI>(a.params, pidx + e, pn);
        if constexpr (EPI == EPI_APPLY) {
          if (a.shadow) a.shadow[pidx + e] = bf16_bits(pn);
        }
      }
    }
  }
}

// Apply: the parameters of one 32-row block of a wave's outputs, as loaded
// (chunk t: 8 elements along a row of a problem stored as is, or down a column
// of one stored transposed), and whether each chunk takes the vector path.
// Every load is issued, so the compiler can count what is in flight: a chunk
// that is not applied reads the launch's descriptors instead (in bounds,
// never used), at a byte offset from the parameters, which keeps it a global
// load.
template <typename T, int TILE, int EPI>
struct ParamBlock {
  static constexpr int CPR = Geo<T, TILE>::HALF / 8;
  static constexpr int NR = 32 * CPR / 64;
  ParamPack<EPI> pq[NR];
  bool pv[NR];
};

template <typename T, int TILE, int EPI>
__device__ __forceinline__ void chunk_at(const ProblemDesc& pd, int ti, int tj, int i, int t, int& gi, int& gj,
                                         int64_t& e) {
  using Gm = Geo<T, TILE>;
  constexpr int HALF = Gm::HALF, CPR = HALF / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gi_w = ti * TILE + (wave >> 1) * HALF, gj_w = tj * TILE + (wave & 1) * HALF;
  const int q = lane + 64 * t;
  if (!pd.transposed) {
    gi = gi_w + i * 32 + q / CPR;
    gj = gj_w + (q % CPR) * 8;
    e = static_cast<int64_t>(gi) * pd.ld + gj;
  } else {
    gi = gi_w + i * 32 + (q & 3) * 8;
    gj = gj_w + (q >> 2);
    e = static_cast<int64_t>(gj) * pd.ld + gi;
  }
}

template <typename T, int TILE, int EPI>
__device__ __forceinline__ void load_param_block(const GemmArgs& a, const ProblemDesc& pd, int ti, int tj, int i,
                                                 ParamBlock<T, TILE, EPI>& b) {
  using PElem = typename std::conditional<EPI == EPI_APPLY_BF16, __bf16, float>::type;
  const char* pbytes = static_cast<const char*>(a.params);
  const int64_t dummy_off = static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.probs) -
                                                 reinterpret_cast<uintptr_t>(a.params));
  const int m = a.m_valid, n = a.n_valid;
#pragma unroll
  for (int t = 0; t < ParamBlock<T, TILE, EPI>::NR; ++t) {
    int gi, gj;
    int64_t e;
    chunk_at<T, TILE, EPI>(pd, ti, tj, i, t, gi, gj, e);
    const bool whole = pd.transposed ? (gj < n && gi + 8 <= m) : (gi < m && gj + 8 <= n);
    b.pv[t] = whole && (((pd.p_base + e) & 7) | ((pd.src_off + e) & 3)) == 0 && e >= pd.lo && e + 8 <= pd.hi;
    b.pq[t].load(reinterpret_cast<const PElem*>(pbytes + (b.pv[t] ? (pd.p_base + e) * int64_t(sizeof(PElem))
                                                                    : dummy_off)));
  }
}

// Epilogue: v = alpha acc + beta D + gamma I, stored (or applied) as the launch asks.
// The beta D term is one explicit fused multiply-add, fma(beta, D, alpha acc), so
// every kernel that forms it rounds it the same way.
// Per wave and per 32-row block i: the accumulators are staged in LDS; a row pass
// gives each lane 8 consecutive columns of several rows (row-major store, or the
// apply of a matrix stored as is), a column pass 8 consecutive rows of one column
// (transposed store, or the apply of a transposed matrix). Every global load of a
// pass (D, params) is issued before any of them is used, and D of block i + 1 is
// requested as soon as block i has consumed its own, so each pass waits for memory
// at most once.
template <typename T, int TILE, bool SYM, int EPI, bool HAS_D>
__device__ __forceinline__ void epilogue(const GemmArgs& a, int prob, int ti, int tj, char* lds0, char* lds1,
                                         f32x16 (&acc)[Geo<T, TILE>::WB][Geo<T, TILE>::WB]) {
  using Gm = Geo<T, TILE>;
  constexpr int HALF = Gm::HALF, WB = Gm::WB, SP = Gm::SP;
  constexpr int CPR = HALF / 8;          // 8-column chunks per staged row
  constexpr int NR = 32 * CPR / 64;      // row-pass tasks per lane
  constexpr int NC = HALF * 4 / 64;      // column-pass tasks per lane
  static_assert(NR == NC, "apply: one chunk count for either pass");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  float* stg = reinterpret_cast<float*>((wave < 2 ? lds0 : lds1) + (wave & 1) * 32 * SP * 4);
  // staged element (row r, column c) of the 32-row block: the column is XORed with
  // 8 * (bits 3-4 of r), which keeps 8-column chunks contiguous and puts the rows
  // r, r + 8, r + 16, r + 24 that one column-pass read gathers in different banks
  auto srow = [&](int r, int c) { return r * SP + (c ^ (((r >> 3) & 3) << 3)); };
  // The mirror of a 16-bit symmetric store goes through a 16-bit copy of the
  // rounded block, laid over the wave's own float staging: row r at byte
  // r * 2 HALF, its 32-byte chunks (16 columns) permuted by h16(r). The row
  // pass writes row r's bytes only after the float rows beneath them have been
  // read (16-bit row r lies below float row r). A transposed read then takes 4
  // rows x 16 columns per 16 lanes; the 8 rows one half wave reads land in 8
  // different chunk slots (HALF = 128) or in 4 slots x 2 row parities (HALF =
  // 64), so each read spreads over all banks.
  constexpr bool TR_MIRROR = sizeof(T) == 2 && SYM && EPI == EPI_STORE;
  constexpr int RP16 = HALF * 2;         // 16-bit staging row pitch (bytes)
  auto h16 = [](int r) {
    if constexpr (HALF == 128) return (r & 3) | (((r >> 3) & 1) << 2);
    else return ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
  };
  auto soff16 = [&](int r, int c) { return r * RP16 + (((c >> 4) ^ h16(r)) << 5) + (c & 15) * 2; };
  char* stg16 = reinterpret_cast<char*>(stg);
  const int gi_w = ti * TILE + wm * HALF;   // first row of this wave's outputs
  const int gj_w = tj * TILE + wn * HALF;   // first column
  const bool diag = SYM && (ti == tj);
  // no element of the tile needs the diagonal tests (the gamma I term, the
  // lower-triangle store): off the diagonal of a symmetric launch, or any tile
  // of a full launch
  const bool plain = !SYM || !diag;   // (full launches have no gamma: the launcher checks)

  int transposed = 0, ld = 0;
  int64_t src = 0, pb = 0, wlo = 0, whi = 0;
  ApplyScalars as{};
  constexpr bool APPLY = (EPI == EPI_APPLY || EPI == EPI_APPLY_BF16);
  ProblemDesc pdv{};
  if constexpr (APPLY) {
    pdv = a.probs[prob];
    transposed = pdv.transposed;
    ld = pdv.ld;
    src = pdv.src_off;
    pb = pdv.p_base;
    wlo = pdv.lo;
    whi = pdv.hi;
    as = ApplyScalars{a.params, a.update_out, a.shadow, a.decay, a.lr};
  }
  // (32-bit iterates: no registers to spare for them; read where used)
  auto scalars = [&]() -> ApplyScalars {
    if constexpr (sizeof(T) == 2) return as;
    else return ApplyScalars{a.params, a.update_out, a.shadow, a.decay, a.lr};
  };
  const int m = a.m_valid, n = a.n_valid;
  // the launch's scalars, read once
  const float alpha = a.alpha, beta = a.beta, gamma = a.gamma;
  const int64_t c_ps = a.c_ps, ct_ps = a.ct_ps, d_ps = a.d_ps;
  const int ldc = a.ldc, ldct = a.ldct, ldd = a.ldd;

  // Store launches always write C; symmetric ones also its mirror Ct, full ones
  // never (the launcher checks both), so the column pass is known at compile time
  T* C = static_cast<T*>(a.C);
  T* Ct = static_cast<T*>(a.Ct);
  const T* D = HAS_D ? static_cast<const T*>(a.D) : nullptr;   // compiled out without a D term
  const bool need_col = APPLY ? (transposed != 0) : SYM;

  Pack8<T> dq[NR];
  auto load_d = [&](int i) {
    if (D == nullptr) return;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int q = lane + 64 * t;
      const int gi = gi_w + i * 32 + q / CPR;
      const int gj = gj_w + (q % CPR) * 8;
      dq[t].load(D + static_cast<int64_t>(prob) * d_ps + static_cast<int64_t>(gi) * ldd + gj);
    }
  };
  load_d(0);

  // Apply: the parameters of the wave's chunks of a 32-row block, as loaded.
  // Block i + 1's are requested before block i's stores: loads and stores
  // share one in-order counter, so a load issued after a store could not be
  // waited for without waiting for the store too.
  // (32-bit iterates: the main loop leaves no room for a second block's
  // parameters, which are then requested right before they are used)
  constexpr bool PF_AHEAD = sizeof(T) == 2;
  constexpr int PEPI = EPI == EPI_STORE ? EPI_APPLY : EPI;
  ParamBlock<T, TILE, PEPI> pblk[2];
  auto chunk = [&](int i, int t, int& gi, int& gj, int64_t& e) { chunk_at<T, TILE, PEPI>(pdv, ti, tj, i, t, gi, gj, e); };
  auto load_params = [&](int i) {
    if constexpr (APPLY) load_param_block<T, TILE, PEPI>(a, pdv, ti, tj, i, pblk[i & 1]);
  };

  // Each wave stages into its own part of LDS, and one wave's LDS accesses are
  // performed in program order, so after the first block (whose staging area the
  // other waves may still be reading operands from) only the compiler has to be
  // kept from reordering them: lds_order().
  auto lds_order = []() { asm volatile("" ::: "memory"); };
#pragma unroll
  for (int i = 0; i < WB; ++i) {
    if (i == 0) {
      __syncthreads();                 // every wave is past its last main-loop LDS read
      if (PF_AHEAD) load_params(0);    // (after the barrier: the main loop's registers are free)
    } else {
      lds_order();
    }
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) stage4(stg + srow(lane & 31, j * 32 + q * 8 + (lane >> 5) * 4), acc[i][j], q);
    lds_order();

    if (!PF_AHEAD) load_params(i);
    else if (i + 1 < WB) load_params(i + 1);   // before this block's stores

    // ---- row pass: each lane finishes one 8-column chunk at a time (and
    // applies it, for a matrix stored as is); the next chunk's staged values
    // are read before this one is finished, so the LDS latency overlaps it
    auto stage_rd = [&](int t, f32x4 (&x)[2]) {
      const int q = lane + 64 * t;
      const int rr = q / CPR, cc = (q % CPR) * 8;
      x[0] = *reinterpret_cast<const f32x4*>(stg + srow(rr, cc));
      x[1] = *reinterpret_cast<const f32x4*>(stg + srow(rr, cc) + 4);
    };
    // A tile off the diagonal of a symmetric launch (and any full launch
    // without a gamma I term) needs no per-element test, so its chunks run as
    // one branch-free block the scheduler can interleave.
    auto row_pass = [&](auto PLAIN) {
      constexpr bool PL = decltype(PLAIN)::value;
      f32x4 sv[2][2];
      stage_rd(0, sv[0]);
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        if (t + 1 < NR) stage_rd(t + 1, sv[(t + 1) & 1]);
        const int q = lane + 64 * t;
        const int rr = q / CPR, cc = (q % CPR) * 8;
        const int gi = gi_w + i * 32 + rr, gj = gj_w + cc;
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = alpha * sv[t & 1][0][e]; v[e + 4] = alpha * sv[t & 1][1][e]; }
        if (D != nullptr) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(beta, dq[t].get(e), v[e]);
        }
        if constexpr (!PL) {
          if (gamma != 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gi == gj + e) v[e] += gamma;
          }
        }
        float4* sp = reinterpret_cast<float4*>(stg + srow(rr, cc));
        if constexpr (APPLY) {
          if (!transposed) {
            // stored m x n: canonical (gi, gj) is local index gi * ld + gj
            if (gi < m && gj < n) {
              const int64_t e = static_cast<int64_t>(gi) * ld + gj;
              apply8<EPI>(scalars(), pb + e, src + e, e, min(8, n - gj), wlo, whi, v, pblk[i & 1].pq[t],
                          pblk[i & 1].pv[t]);
            }
          } else {
            // the value goes back to the staging area for the column pass
            sp[0] = make_float4(v[0], v[1], v[2], v[3]);
            sp[1] = make_float4(v[4], v[5], v[6], v[7]);
          }
        } else {
          T o[8];
          rne<T, 8>(v, o);
          T* cp = C + static_cast<int64_t>(prob) * c_ps + static_cast<int64_t>(gi) * ldc + gj;
          if (PL || !diag || gi >= gj + 7) {
            st8<T>(cp, o);
          } else {
            for (int e = 0; e < 8; ++e)
              if (gi >= gj + e) cp[e] = o[e];
          }
          if constexpr (TR_MIRROR) {
            u16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = __builtin_bit_cast(unsigned short, o[e]);
            *reinterpret_cast<u16x8*>(stg16 + soff16(rr, cc)) = w;
          } else if (need_col) {
            sp[0] = make_float4(to_f32(o[0]), to_f32(o[1]), to_f32(o[2]), to_f32(o[3]));
            sp[1] = make_float4(to_f32(o[4]), to_f32(o[5]), to_f32(o[6]), to_f32(o[7]));
          }
        }
      }
    };
    if constexpr (!SYM) row_pass(std::true_type{});
    else if (plain) row_pass(std::true_type{});
    else row_pass(std::false_type{});
    if (i + 1 < WB) load_d(i + 1);

    // ---- column pass
    if (need_col) {
      lds_order();
      if constexpr (APPLY) {
        // stored n x m: canonical (gi, gj) is local index gj * ld + gi
#pragma unroll
        for (int t = 0; t < NC; ++t) {
          int gi, gj;
          int64_t e;
          chunk(i, t, gi, gj, e);
          const int q = lane + 64 * t;
          const int r8 = (q & 3) * 8, cc = q >> 2;
          if (gj < n && gi < m) {
            float w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = stg[srow(r8 + u, cc)];
            apply8<EPI>(scalars(), pb + e, src + e, e, min(8, m - gi), wlo, whi, w, pblk[i & 1].pq[t], pblk[i & 1].pv[t]);
          }
        }
      } else {
        auto col_pass = [&](auto PLAIN) {
          constexpr bool PL = decltype(PLAIN)::value;
          if constexpr (TR_MIRROR) {
            // lane (g, s) = (lane / 16, lane % 16): rows 8g .. 8g + 7 of column
            // 16t + s, two transposed reads of 4 rows each
            const int g = lane >> 4, s16 = lane & 15;
            const int r0 = 8 * g + (s16 >> 2);
#pragma unroll
            for (int t = 0; t < NC; ++t) {
              const int c0 = 16 * t + 4 * (s16 & 3);
              const u16x4 lo = __builtin_bit_cast(u16x4, TrRead<T>::get(stg16 + soff16(r0, c0)));
              const u16x4 hi = __builtin_bit_cast(u16x4, TrRead<T>::get(stg16 + soff16(r0 + 4, c0)));
              const int gi = gi_w + i * 32 + 8 * g, gj = gj_w + 16 * t + s16;
              const u16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              unsigned short* cp = reinterpret_cast<unsigned short*>(Ct + static_cast<int64_t>(prob) * ct_ps +
                                                                     static_cast<int64_t>(gj) * ldct + gi);
              if (PL || !diag || gi > gj) {
                *reinterpret_cast<u16x8*>(cp) = w;
              } else {
                for (int e = 0; e < 8; ++e)
                  if (gi + e > gj) cp[e] = w[e];
              }
            }
            return;
          }
#pragma unroll
          for (int t = 0; t < NC; ++t) {
            const int q = lane + 64 * t;
            const int r8 = (q & 3) * 8, cc = q >> 2;
            const int gi = gi_w + i * 32 + r8, gj = gj_w + cc;
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = stg[srow(r8 + e, cc)];
            T o[8];
            rne<T, 8>(w, o);
            T* cp = Ct + static_cast<int64_t>(prob) * ct_ps + static_cast<int64_t>(gj) * ldct + gi;
            if (PL || !diag || gi > gj) {
              st8<T>(cp, o);
            } else {
              for (int e = 0; e < 8; ++e)
                if (gi + e > gj) cp[e] = o[e];
            }
          }
        };
        if (plain) col_pass(std::true_type{});   // (symmetric launches only)
        else col_pass(std::false_type{});
      }
    }
  }
}

// One launch covers up to kBatchGroups shape groups: block b belongs to the last
// group g with start[g] <= b. HAS_D: the launch has a beta D term (every group
// of it); without, the epilogue is compiled with no D code at all.
template <typename T, int TILE, bool SYM, int EPI, bool NN, bool HAS_D>
__global__ __launch_bounds__(256) void ns_gemm(GemmBatch batch) {
  using Gm = Geo<T, TILE>;
  __shared__ __attribute__((aligned(1024))) char lds0[2 * Gm::OPB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * Gm::OPB];
  const int bid = static_cast<int>(blockIdx.x);
  int g = 0;
#pragma unroll
  for (int q = 1; q < kBatchGroups; ++q)
    if (q < batch.n && bid >= batch.start[q]) g = q;
  const GemmArgs& a = batch.g[g];
  int prob, ti, tj;
  decode_tile<SYM>(a, bid - batch.start[g], prob, ti, tj);
  f32x16 acc[Gm::WB][Gm::WB];
  mainloop<T, TILE, NN>(a, prob, ti, tj, lds0, lds1, acc);
  epilogue<T, TILE, SYM, EPI, HAS_D>(a, prob, ti, tj, lds0, lds1, acc);
}

// ---------------------------------------------------------------------------
// Groups with a single tile row (m <= 128, 16-bit iterates): the update
// X' = B X and the next Gram matrix A' = X' X'^T in one pass.
//
// One workgroup per problem keeps B in LDS and streams X one 128-column tile at a
// time: each tile is the K x N operand of B X, so X is read once; X' goes out to HBM and, rounded as stored, into LDS, where it is
// the operand of the tile's contribution to X' X'^T, accumulated in registers
// over all tiles. Every output element sees the same products in the same k
// order as the separate update and X X^T launches, so the results are
// bit-identical to theirs.
//
// Arguments: P = B (mp x mp, the a I term included), Q = X (mp x np), C = X',
// Ct = A' (mp x mp, stored symmetric); alpha as in the update (no D term);
// tiles_n = np / 128.
template <typename T>
__global__ __launch_bounds__(256) void ns_update_gram(GemmBatch batch) {
  using Gm = Geo<T, 128>;
  static_assert(sizeof(T) == 2, "16-bit iterates only");
  constexpr int HALF = Gm::HALF, WB = Gm::WB, SP = Gm::SP;   // 64, 2, 68
  constexpr int KS = 64;                                      // K elements per slice
  constexpr int RB = 256;                                     // bytes of one X row of a tile
  constexpr int SLB = 128 * 128;                              // bytes of one K-contiguous slice plane
  constexpr int XSB = KS * RB;                                // bytes of one NN slice of an X tile
  constexpr int STG = 32 * SP * 4;                            // epilogue staging bytes per wave
  __shared__ __attribute__((aligned(1024))) char Bs[2 * SLB];      // B, K-contiguous, two slices
  __shared__ __attribute__((aligned(1024))) char Xs[2 * XSB];      // X tile, K x N, two slices
  __shared__ __attribute__((aligned(1024))) char Ns[2 * SLB];      // X' tile, K-contiguous planes
  __shared__ __attribute__((aligned(1024))) char St[4 * STG];      // epilogue staging

  const int bid = static_cast<int>(blockIdx.x);
  int g = 0;
#pragma unroll
  for (int q = 1; q < kBatchGroups; ++q)
    if (q < batch.n && bid >= batch.start[q]) g = q;
  const GemmArgs& a = batch.g[g];
  const int prob = bid - batch.start[g];
  const int NT = a.tiles_n;

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  using V = typename Gm::V;

  // ---- B into LDS (row r = (wave * 4 + it) * 8 + lane / 8, chunk lane % 8 of slice sl)
  {
    const char* Bg = static_cast<const char*>(a.P) + static_cast<int64_t>(prob) * a.p_ps * 2;
    u16x8 rb[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int sl = v >> 2, r = (wave * 4 + (v & 3)) * 8 + (lane >> 3), c = lane & 7;
      rb[v] = *reinterpret_cast<const u16x8*>(Bg + static_cast<int64_t>(r) * a.ldp * 2 + sl * 128 + c * 16);
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int sl = v >> 2, r = (wave * 4 + (v & 3)) * 8 + (lane >> 3), c = lane & 7;
      *reinterpret_cast<u16x8*>(Bs + sl * SLB + r * 128 + ((c ^ swz(r)) << 4)) = rb[v];
    }
  }

  // ---- X tile loads: thread t covers chunk (it * 256 + t) of slice it / 4, i.e. row
  // kr = (it % 4) * 16 + t / 16 of that slice, 16-byte chunk t % 16
  const char* Xg = static_cast<const char*>(a.Q) + static_cast<int64_t>(prob) * a.q_ps * 2;
  int xofs[8];
  int64_t xsrc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int sl = v >> 2, id = (v & 3) * 256 + tid, kr = id >> 4, c = id & 15;
    xsrc[v] = (static_cast<int64_t>(sl * KS + kr) * a.ldq) * 2 + c * 16;
    xofs[v] = sl * XSB + kr * RB + (((c >> 1) ^ nn_swz(kr)) << 5) + ((c & 1) << 4);
  }
  auto xload = [&](u16x8 (&r)[8], int jt) {
    const int64_t col = static_cast<int64_t>(jt) * 128 * 2;
#pragma unroll
    for (int v = 0; v < 8; ++v) r[v] = *reinterpret_cast<const u16x8*>(Xg + xsrc[v] + col);
  };
  auto xwrite = [&](const u16x8 (&r)[8]) {
#pragma unroll
    for (int v = 0; v < 8; ++v) *reinterpret_cast<u16x8*>(Xs + xofs[v]) = r[v];
  };

  // ---- MFMA operand offsets: K-contiguous planes (B, X') and the NN X tile
  int aoff[WB][4], boff[WB][4], bnn[WB][2];
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
#pragma unroll
  for (int j = 0; j < WB; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int gq = lane >> 4, sl = lane & 15;
      const int kr = 8 * (gq >> 1) + 4 * h + (sl >> 2);
      const int cb = (wn * HALF + j * 32 + 16 * (gq & 1) + 4 * (sl & 3)) * 2;
      bnn[j][h] = kr * RB + (((cb >> 5) ^ nn_swz(kr)) << 5) + (cb & 31);
    }

  f32x16 accA[WB][WB], accC[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) accA[i][j][r] = 0.0f;

  float* stg = reinterpret_cast<float*>(St + wave * STG);
  auto srow = [&](int r, int c) { return r * SP + (c ^ (((r >> 3) & 3) << 3)); };
  T* Cg = static_cast<T*>(a.C) + static_cast<int64_t>(prob) * a.c_ps;

  auto tile = [&](u16x8 (&r)[8], int jt) {
    xwrite(r);
    __syncthreads();                       // X tile (and, first time, B) in LDS; last Gram reads done
    if (jt + 3 < NT) xload(r, jt + 3);     // three tiles in flight (two: 0.5% slower steps)

    // X'_tile = B X_tile over K = 128 (two slices, four sub-steps each)
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) accC[i][j][e] = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        V xa[WB], xb[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) xa[i] = *reinterpret_cast<const V*>(Bs + sl * SLB + aoff[i][ks]);
#pragma unroll
        for (int j = 0; j < WB; ++j) {
          const char* base = Xs + sl * XSB + ks * 16 * RB;
          const auto lo = TrRead<T>::get(base + bnn[j][0]);
          const auto hi = TrRead<T>::get(base + bnn[j][1]);
          xb[j] = __builtin_bit_cast(V, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j) Mfma<T>::run(xb[j], xa[i], accC[i][j]);
      }

    // epilogue: v = alpha acc, rounded; to HBM and to the K-contiguous planes of X'
#pragma unroll
    for (int i = 0; i < WB; ++i) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) stage4(stg + srow(lane & 31, j * 32 + q * 8 + (lane >> 5) * 4), accC[i][j], q);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int q = lane + 64 * t;
        const int rr = q >> 3, cc = (q & 7) * 8;
        const int gi = wm * HALF + i * 32 + rr, gj = wn * HALF + cc;   // row (= k of X), column in tile
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(stg + srow(rr, cc));
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(stg + srow(rr, cc) + 4);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = a.alpha * (e < 4 ? s0[e] : s1[e - 4]);
        T o[8];
        rne<T, 8>(v, o);
        st8<T>(Cg + static_cast<int64_t>(gi) * a.ldc + static_cast<int64_t>(jt) * 128 + gj, o);
        const int pl = gj >> 6, c = (gj & 63) >> 3;
        u16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = __builtin_bit_cast(unsigned short, o[e]);
        *reinterpret_cast<u16x8*>(Ns + pl * SLB + gi * 128 + ((c ^ swz(gi)) << 4)) = w;
      }
    }
    __syncthreads();                       // X' planes complete; X tile no longer read

    // A' += X'_tile X'_tile^T over the tile's 128 columns
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        V xa[WB], xb[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) xa[i] = *reinterpret_cast<const V*>(Ns + pl * SLB + aoff[i][ks]);
#pragma unroll
        for (int j = 0; j < WB; ++j) xb[j] = *reinterpret_cast<const V*>(Ns + pl * SLB + boff[j][ks]);
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j) Mfma<T>::run(xb[j], xa[i], accA[i][j]);
      }
  };

  u16x8 r0[8], r1[8], r2[8];
  xload(r0, 0);
  if (NT > 1) xload(r1, 1);
  if (NT > 2) xload(r2, 2);
  for (int jt = 0; jt < NT; jt += 3) {
    tile(r0, jt);
    if (jt + 1 < NT) tile(r1, jt + 1);
    if (jt + 2 < NT) tile(r2, jt + 2);
  }

  // A' stored symmetric (lower triangle, mirrored), as the X X^T launch stores it
  GemmArgs s{};
  s.C = a.Ct; s.c_ps = a.ct_ps; s.ldc = a.ldct;
  s.Ct = a.Ct; s.ct_ps = a.ct_ps; s.ldct = a.ldct;
  s.alpha = 1.0f;
  epilogue<T, 128, true, EPI_STORE, false>(s, prob, 0, 0, St, St + 2 * STG, accA);
}

hipError_t launch_update_gram(int dtype, const GemmBatch& b, hipStream_t s) {
  if (b.n < 1 || b.n > kBatchGroups || b.start[0] != 0) return hipErrorInvalidValue;
  for (int g = 0; g < b.n; ++g) {
    const GemmArgs& a = b.g[g];
    if (a.K != 128 || a.tiles_n < 1 || b.start[g + 1] - b.start[g] != a.total_tiles) return hipErrorInvalidValue;
    if (a.D != nullptr || a.beta != 0.0f) return hipErrorInvalidValue;   // no D term
  }
  if (b.start[b.n] <= 0) return hipSuccess;
  switch (dtype) {
    case MUON_DTYPE_BF16:
      hipLaunchKernelGGL(ns_update_gram<__bf16>, dim3(b.start[b.n]), dim3(256), 0, s, b);
      break;
    case MUON_DTYPE_F16:
      hipLaunchKernelGGL(ns_update_gram<_Float16>, dim3(b.start[b.n]), dim3(256), 0, s, b);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Single-tile-row groups (m <= 128, fp16), Gram method: the chain on the small
// matrices, one workgroup per problem.
//
// R, Q, T and P (128 x 128 fp16, 32 KiB each) stay in LDS for every step, each
// as two K planes of 128-byte rows, 16-byte chunks XOR-swizzled by the row (the
// layout the MFMA operand reads of the other kernels use). Every product is
// NT: R, Q and T are stored symmetric, so a row is also a column, and P is kept
// transposed (rows of P^T) while it is the right operand of Q P; the last P is
// stored as is, the left operand of P X0. Each product runs the MFMAs of the
// 128-tile launch in the same k order and finishes with the same epilogue
// arithmetic, then stores straight from the accumulators: a lane holds four
// consecutive rows of one column, one 8-byte write of the transposed position,
// plus 2-byte writes where the row-major position is needed (the mirror of a
// symmetric result, and the last P), which is then copied out row-major for the
// apply launch. (Fused here, the apply streamed X0 and the parameters from one
// workgroup per CU, about 40% slower than its own launch with two.)
template <typename T>
__global__ __launch_bounds__(256) void gram_chain_kernel(GramChainBatch batch) {
  using Gm = Geo<T, 128>;
  static_assert(sizeof(T) == 2, "16-bit iterates only");
  constexpr int WB = Gm::WB, HALF = Gm::HALF;                 // 2, 64
  constexpr int PL = 128 * 128;                               // bytes of one K plane
  constexpr int MAT = 2 * PL;                                 // bytes of one matrix
  __shared__ __attribute__((aligned(1024))) char L[4 * MAT];
  __shared__ __attribute__((aligned(16))) char Dump[64 * 2];
  char* const Rm = L;
  char* const Qm = L + MAT;
  char* const Tm = L + 2 * MAT;
  char* const Pm = L + 3 * MAT;

  const int bid = static_cast<int>(blockIdx.x);
  int g = 0;
#pragma unroll
  for (int q = 1; q < kBatchGroups; ++q)
    if (q < batch.n && bid >= batch.start[q]) g = q;
  const GramChainArgs& a = batch.g[g];
  const int prob = bid - batch.start[g];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  using V = typename Gm::V;

  // byte offset of element (r, k) of a matrix held as K planes
  auto at = [](int r, int k) { return (k >> 6) * PL + r * 128 + ((((k & 63) >> 3) ^ swz(r)) << 4) + (k & 7) * 2; };

  // ---- R0 (row-major, pitch 128) into R
  {
    const char* Rg = static_cast<const char*>(a.R0) + static_cast<int64_t>(prob) * a.r_ps * 2;
    u16x8 rb[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int id = v * 256 + tid, r = id >> 4, c = id & 15;
      rb[v] = *reinterpret_cast<const u16x8*>(Rg + r * 256 + c * 16);
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int id = v * 256 + tid, r = id >> 4, c = id & 15;
      *reinterpret_cast<u16x8*>(Rm + (c >> 3) * PL + r * 128 + (((c & 7) ^ swz(r)) << 4)) = rb[v];
    }
  }

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
  // acc = A B^T over K = 128: A and B rows from LDS planes, k in increasing order
  auto product = [&](const char* A, const char* B) {
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // every operand of the product is requested before the first MFMA (one wave
    // per SIMD: the registers are there, and the reads overlap the MFMAs)
    V xa[8][WB], xb[8][WB];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int pl = t >> 2, ks = t & 3;
#pragma unroll
      for (int i = 0; i < WB; ++i) xa[t][i] = *reinterpret_cast<const V*>(A + pl * PL + aoff[i][ks]);
#pragma unroll
      for (int j = 0; j < WB; ++j) xb[t][j] = *reinterpret_cast<const V*>(B + pl * PL + boff[j][ks]);
    }
    __builtin_amdgcn_sched_barrier(0);             // keep the reads ahead of the MFMAs
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) Mfma<T>::run(xa[t][i], xb[t][j], acc[i][j]);
  };
  // accumulator element (block i, j; register q * 4 + e) is row row0 + e, column
  // col. The stores take the lane index through an opaque copy made per call:
  // their many LDS addresses do not depend on the step, and hoisted out of the
  // step loop they would all stay live at once.
  auto opaque_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto row0_of = [&](int ln, int i, int q) { return wm * HALF + i * 32 + q * 8 + (ln >> 5) * 4; };
  auto col_of = [&](int ln, int j) { return wn * HALF + j * 32 + (ln & 31); };

  // symmetric store of v = alpha acc + beta D + gamma I (D symmetric or none), as
  // the symmetric launch stores it: the lower triangle (row >= column) of the
  // accumulators, rounded, at its place and mirrored
  auto store_sym = [&](char* dst, float alpha, float beta, const char* D, float gamma) {
    const int ln = opaque_lane();
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j) {
        // 32 x 32 block (br, bc) of the matrix, the same for the whole wave:
        // above the diagonal nothing is stored; below it every element is
        // strictly lower; only diagonal blocks test element by element
        const int br = wm * WB + i, bc = wn * WB + j;
        if (br < bc) continue;
        const int col = col_of(ln, j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row0 = row0_of(ln, i, q);
          float v[4];
          u16x4 dv;
          if (D != nullptr) dv = *reinterpret_cast<const u16x4*>(D + at(col, row0));   // D[row][col] = D[col][row]
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = alpha * acc[i][j][q * 4 + e];
            if (D != nullptr) v[e] = __builtin_fmaf(beta, static_cast<float>(__builtin_bit_cast(T, (unsigned short)dv[e])), v[e]);
            if (br == bc) v[e] = (gamma != 0.0f && row0 + e == col) ? v[e] + gamma : v[e];
          }
          T r[4];
          rne<T, 4>(v, r);
          u16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(unsigned short, r[e]);
          if (br > bc) {
            *reinterpret_cast<u16x4*>(dst + at(col, row0)) = o;          // (col, row0 + e): mirror
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<unsigned short*>(dst + at(row0 + e, col)) = o[e];
          } else {
            // diagonal block: an element that is not stored goes to the lane's
            // own slot of a dump area instead (no divergent branches)
            char* const dump = Dump + ln * 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              *reinterpret_cast<unsigned short*>(row0 + e >= col ? dst + at(col, row0 + e) : dump) = o[e];
              *reinterpret_cast<unsigned short*>(row0 + e > col ? dst + at(row0 + e, col) : dump) = o[e];
            }
          }
        }
      }
  };
  // full store of the rounded accumulators: transposed (row col holds column
  // col) or as is
  auto store_full = [&](char* dst, bool transposed) {
    const int ln = opaque_lane();
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j) {
        const int col = col_of(ln, j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row0 = row0_of(ln, i, q);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = 1.0f * acc[i][j][q * 4 + e];
          T r[4];
          rne<T, 4>(v, r);
          u16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(unsigned short, r[e]);
          if (transposed) {
            *reinterpret_cast<u16x4*>(dst + at(col, row0)) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<unsigned short*>(dst + at(row0 + e, col)) = o[e];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  __syncthreads();                                 // R0 in LDS
  const int S = a.steps;
  for (int k = 0; k < S; ++k) {
    product(Rm, Rm);                               // Q = qa I + qb R + qc R R
    store_sym(Qm, a.qc, a.qb, Rm, a.qa);
    if (k == 0) store_sym(Pm, a.qc, a.qb, Rm, a.qa);   // P = Q (symmetric: also P^T)
    __syncthreads();
    if (k > 0) {                                   // P <- Q P, P^T as the right operand
      product(Qm, Pm);
      __syncthreads();                             // every read of the old P done
      store_full(Pm, k < S - 1);
    }
    if (k < S - 1) {
      product(Rm, Qm);                             // T = R Q (Q symmetric)
      store_sym(Tm, 1.0f, 0.0f, nullptr, 0.0f);
      __syncthreads();
      product(Qm, Tm);                             // R <- Q T (T symmetric); R is not read here
      store_sym(Rm, 1.0f, 0.0f, nullptr, 0.0f);
    }
    __syncthreads();
  }

  // ---- the final P (row-major in LDS) out, row-major with pitch 128
  {
    char* Pg = static_cast<char*>(a.P) + static_cast<int64_t>(prob) * a.p_ps * 2;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int id = v * 256 + tid, r = id >> 4, c = id & 15;
      *reinterpret_cast<u16x8*>(Pg + r * 256 + c * 16) =
          *reinterpret_cast<const u16x8*>(Pm + (c >> 3) * PL + r * 128 + (((c & 7) ^ swz(r)) << 4));
    }
  }
}

hipError_t launch_gram_chain(int dtype, const GramChainBatch& b, hipStream_t s) {
  if (b.n < 1 || b.n > kBatchGroups || b.start[0] != 0) return hipErrorInvalidValue;
  for (int g = 0; g < b.n; ++g) {
    const GramChainArgs& a = b.g[g];
    if (a.steps < 1 || a.count < 0 || b.start[g + 1] - b.start[g] != a.count) return hipErrorInvalidValue;
  }
  if (b.start[b.n] <= 0) return hipSuccess;
  if (dtype != MUON_DTYPE_F16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gram_chain_kernel<_Float16>, dim3(b.start[b.n]), dim3(256), 0, s, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Single-tile-row groups (m <= 128, 16-bit iterates): X0 and its Gram matrix
// R = alpha X0 X0^T in one pass.
//
// One workgroup per problem streams the momentum one 128-column tile of X0 at a
// time: it forms X0 = round(M * inv_norm) exactly as the X0 kernel does (a matrix
// stored transposed is turned in LDS), writes it to HBM and into LDS, and adds the
// tile's contribution to X0 X0^T in registers; the next tile's momentum is loaded
// while the current one's products run. The products and their k order are those
// of the symmetric launch, so X0 and R are bit-identical to the separate kernels.
template <typename T>
__global__ __launch_bounds__(256) void prep_gram_kernel(PrepGramArgs a) {
  using Gm = Geo<T, 128>;
  static_assert(sizeof(T) == 2, "16-bit iterates only");
  constexpr int WB = Gm::WB, HALF = Gm::HALF, SP = Gm::SP;   // 2, 64, 68
  constexpr int SLB = 128 * 128;                              // bytes of one K-contiguous plane
  constexpr int MP = 129;                                     // pitch (floats) of the transpose tile
  constexpr int STG = 32 * SP * 4;                            // epilogue staging bytes per wave
  static_assert(4 * STG <= 128 * MP * 4, "epilogue staging fits in the transpose tile");
  __shared__ __attribute__((aligned(1024))) float Ms[128 * MP];   // transpose tile, then staging
  __shared__ __attribute__((aligned(1024))) char Ns[2 * SLB];     // X0 tile, K-contiguous planes

  const int p = static_cast<int>(blockIdx.x);
  const ProblemDesc pd = a.probs[p];
  const float inv = a.inv_norm[p];
  const int m = a.m, n = a.n, NT = a.np / 128;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r = tid >> 1, hh = tid & 1;   // this thread's row (or stored row) and half of it
  using V = typename Gm::V;

  // raw momentum of tile jt for this thread: 64 consecutive stored elements
  auto load = [&](float (&buf)[64], int jt) {
    int64_t base;
    bool ok, vec;
    if (!pd.transposed) {                 // row r, columns jt*128 + hh*64 ..
      const int k0 = jt * 128 + hh * 64;
      base = pd.src_off + static_cast<int64_t>(r) * pd.ld + k0;
      ok = r < m;
      vec = ok && k0 + 64 <= n && (base & 3) == 0;
#pragma unroll
      for (int e = 0; e < 64; e += 4) {
        if (vec) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(a.M + base + e);
          buf[e] = w[0]; buf[e + 1] = w[1]; buf[e + 2] = w[2]; buf[e + 3] = w[3];
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) buf[e + u] = (ok && k0 + e + u < n) ? a.M[base + e + u] : 0.0f;
        }
      }
    } else {                              // stored row jt*128 + r, elements hh*64 ..
      const int kk = jt * 128 + r, i0 = hh * 64;
      base = pd.src_off + static_cast<int64_t>(kk) * pd.ld + i0;
      ok = kk < n;
      vec = ok && i0 + 64 <= m && (base & 3) == 0;
#pragma unroll
      for (int e = 0; e < 64; e += 4) {
        if (vec) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(a.M + base + e);
          buf[e] = w[0]; buf[e + 1] = w[1]; buf[e + 2] = w[2]; buf[e + 3] = w[3];
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) buf[e + u] = (ok && i0 + e + u < m) ? a.M[base + e + u] : 0.0f;
        }
      }
    }
  };

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
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  T* Xg = static_cast<T*>(a.X) + static_cast<int64_t>(p) * a.mp * a.np;
  auto tile = [&](float (&buf)[64], int jt) {
    // X0 row r, columns hh*64 .. of the tile (through LDS when stored transposed)
    float v[64];
    if (pd.transposed) {
#pragma unroll
      for (int e = 0; e < 64; ++e) Ms[(hh * 64 + e) * MP + r] = buf[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 64; ++e) v[e] = Ms[r * MP + hh * 64 + e] * inv;
    } else {
#pragma unroll
      for (int e = 0; e < 64; ++e) v[e] = buf[e] * inv;
    }
    T* dst = Xg + static_cast<int64_t>(r) * a.np + jt * 128 + hh * 64;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = v[c * 8 + e];
      T rx[8];
      rne<T, 8>(x, rx);
      u16x8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = __builtin_bit_cast(unsigned short, rx[e]);
      *reinterpret_cast<u16x8*>(dst + c * 8) = w;
      *reinterpret_cast<u16x8*>(Ns + hh * SLB + r * 128 + ((c ^ swz(r)) << 4)) = w;
    }
    __syncthreads();                       // X0 tile complete in LDS; transpose tile read
    if (jt + 1 < NT) load(buf, jt + 1);

    // R += X0_tile X0_tile^T over the tile's 128 columns
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        V xa[WB], xb[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) xa[i] = *reinterpret_cast<const V*>(Ns + pl * SLB + aoff[i][ks]);
#pragma unroll
        for (int j = 0; j < WB; ++j) xb[j] = *reinterpret_cast<const V*>(Ns + pl * SLB + boff[j][ks]);
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j) Mfma<T>::run(xb[j], xa[i], acc[i][j]);
      }
    __syncthreads();                       // products done before the tile buffers are reused
  };
  float buf[64];
  load(buf, 0);
  for (int jt = 0; jt < NT; ++jt) tile(buf, jt);

  GemmArgs s{};
  s.C = a.R; s.c_ps = static_cast<int64_t>(a.mp) * a.mp; s.ldc = a.mp;
  s.Ct = a.R; s.ct_ps = s.c_ps; s.ldct = a.mp;
  s.alpha = a.alpha;
  char* st = reinterpret_cast<char*>(Ms);
  epilogue<T, 128, true, EPI_STORE, false>(s, p, 0, 0, st, st + 2 * STG, acc);
}

hipError_t launch_prep_gram(int dtype, const PrepGramArgs& a, hipStream_t s) {
  if (a.n_problems <= 0) return hipSuccess;
  if (a.mp != 128 || a.m < 1 || a.m > 128 || a.np % 128 != 0 || a.n > a.np) return hipErrorInvalidValue;
  switch (dtype) {
    case MUON_DTYPE_BF16:
      hipLaunchKernelGGL(prep_gram_kernel<__bf16>, dim3(a.n_problems), dim3(256), 0, s, a);
      break;
    case MUON_DTYPE_F16:
      hipLaunchKernelGGL(prep_gram_kernel<_Float16>, dim3(a.n_problems), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers

template <typename T, int TILE, bool SYM, int EPI, bool NN, bool HAS_D>
static hipError_t launch_t(const GemmBatch& b, hipStream_t s) {
  if (b.n < 1 || b.n > kBatchGroups) return hipErrorInvalidValue;
  for (int g = 0; g < b.n; ++g) {
    const GemmArgs& a = b.g[g];
    // the main loop runs whole pairs of 128-byte K slices
    if (a.K <= 0 || a.K % (2 * 128 / static_cast<int>(sizeof(T))) != 0) return hipErrorInvalidValue;
    if (b.start[g + 1] - b.start[g] != a.total_tiles || a.total_tiles < 0) return hipErrorInvalidValue;
    if ((a.D != nullptr) != HAS_D) return hipErrorInvalidValue;   // one kind of epilogue per launch
    if (!SYM && a.gamma != 0.0f) return hipErrorInvalidValue;      // gamma I: symmetric launches only
    // store launches write C, and its mirror Ct exactly when symmetric
    if (EPI == EPI_STORE && (a.C == nullptr || (a.Ct != nullptr) != SYM)) return hipErrorInvalidValue;
  }
  if (b.start[0] != 0 || b.start[b.n] <= 0) return b.start[b.n] == 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL((ns_gemm<T, TILE, SYM, EPI, NN, HAS_D>), dim3(b.start[b.n]), dim3(256), 0, s, b);
  return hipGetLastError();
}

// Symmetric launches take both operands K-contiguous (NT), with or without a D
// term; full launches take the second operand stored K x N (NN) and have none.
template <typename T, int TILE>
static hipError_t launch_tile(bool sym, int epi, const GemmBatch& b, hipStream_t s) {
  if (sym) {
    if (epi != EPI_STORE) return hipErrorInvalidValue;
    return b.g[0].D != nullptr ? launch_t<T, TILE, true, EPI_STORE, false, true>(b, s)
                               : launch_t<T, TILE, true, EPI_STORE, false, false>(b, s);
  }
  if (epi == EPI_APPLY) return launch_t<T, TILE, false, EPI_APPLY, true, false>(b, s);
  if (epi == EPI_APPLY_BF16) return launch_t<T, TILE, false, EPI_APPLY_BF16, true, false>(b, s);
  return launch_t<T, TILE, false, EPI_STORE, true, false>(b, s);
}

template <typename T>
static hipError_t launch_dtype(int tile, bool sym, int epi, const GemmBatch& b, hipStream_t s) {
  return tile == 256 ? launch_tile<T, 256>(sym, epi, b, s) : launch_tile<T, 128>(sym, epi, b, s);
}

hipError_t launch_ns_gemm(int dtype, int tile, bool sym, int epi, const GemmBatch& b, hipStream_t s) {
  switch (dtype) {
    case MUON_DTYPE_BF16: return launch_dtype<__bf16>(tile, sym, epi, b, s);
    case MUON_DTYPE_F16: return launch_dtype<_Float16>(tile, sym, epi, b, s);
    default: return launch_dtype<float>(tile, sym, epi, b, s);
  }
}

}  // namespace muon
