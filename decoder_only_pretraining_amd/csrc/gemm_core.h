// bf16 MFMA GEMM core for gfx950: C[M][N] = sum_k A(m,k) * B(n,k), fp32
// accumulation, templated on the block tile, the operand layouts, operand
// prologues and the output epilogue.
//
// Operand layouts. A "K-major" operand stores rows of the contraction index
// (row m holds A(m, k) contiguously); an "MN-major" operand stores rows of
// the output index (row k holds A(m, k) contiguously). Activations enter the
// weight-gradient products MN-major (the contraction runs over tokens).
//
// LDS. K-major tiles are kept as [rows][BK] with 16-byte granules XOR-
// swizzled by row, so both the global->LDS writes and the MFMA fragment
// reads (one 16-byte read per lane) are free of bank conflicts. MN-major
// tiles are kept as they are in memory, [BK][rows + 32] (the pad spreads
// four consecutive k rows over all 64 banks), and fragments are read with
// the gfx950 transposing LDS load ds_read_b64_tr_b16: within a 16-lane
// group, source lane 4q + a addresses T[k0 + q][m0 + 4a .. +3] and output
// lane i receives T[k0 .. k0 + 3][m0 + i], i.e. four consecutive
// contraction slots of one output row. Two such loads make the 8-slot
// fragment of v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 4 wavefronts in a 2x2 grid; each wavefront owns a
// (BM/2) x (BN/2) accumulator tile of 32x32 MFMA blocks. Two LDS stages:
// stage k+1 streams in while the MFMAs of stage k run. When both operands
// are K-major the fill uses direct global->LDS loads (no VGPR staging, no
// ds_write: on gfx950 the ds_write bandwidth is about half the ds_read
// bandwidth); products with an MN-major operand measured faster with the
// register-staged fill, stored after the stage's MFMAs. The
// epilogue reuses the LDS to turn the MFMA accumulator layout (four rows by
// one column per lane) into row-contiguous 4-column vectors for the global
// stores and the loads of epilogue operands.
//
// Grid: blockIdx.x enumerates (K split, output tile) pairs, split-major.
// Tile order is XCD-aware: the dispatcher deals consecutive workgroups to
// the 8 XCDs in turn, so the linear id is remapped to give each XCD a
// contiguous range of one split's tiles, walked in groups of 8 tile rows
// that share B panels in its L2.
#pragma once
#include "device_common.h"

#include <type_traits>

namespace gk {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct alignas(16) U128 {
  uint32_t w[4];
};

template <int ROWS, int BK, bool KMAJ>
struct TileGeom {
  static constexpr int G = BK / 8;               // 16-byte granules per K-major row
  static constexpr int RPS = 16 / G;             // K-major rows per 256 bytes
  static constexpr int PITCH = ROWS + 32;        // MN-major row pitch (elements)
  static constexpr int ELEMS = KMAJ ? ROWS * BK : BK * PITCH;
  static constexpr int NV = ROWS * BK / 8 / 256; // 16-byte vectors per thread per stage
  static_assert(NV >= 1, "tile too small");
  __device__ static __forceinline__ int kmaj_off(int r, int g) {
    return r * BK + ((g ^ ((r / RPS) & (G - 1))) << 3);
  }
};

// Register-staged stage fill by NTHR threads (NV 16-byte vectors each).
template <int ROWS, int BK, bool KMAJ, int NTHR = 256>
struct Loader {
  using Geo = TileGeom<ROWS, BK, KMAJ>;
  static constexpr int NV = ROWS * BK / 8 / NTHR;
  static_assert(NV >= 1 && ROWS * BK / 8 % NTHR == 0, "whole vectors per thread");
  U128 raw[NV];
  bool ok[NV];

  __device__ __forceinline__ void load(const bf16* __restrict__ p, int64_t ld, int64_t mn0,
                                       int64_t MN, int64_t k0, int64_t khi, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NTHR;
      int64_t mn, k;
      if (KMAJ) {
        mn = mn0 + v / Geo::G;
        k = k0 + (v % Geo::G) * 8;
      } else {
        k = k0 + v / (ROWS / 8);
        mn = mn0 + (v % (ROWS / 8)) * 8;
      }
      ok[i] = (mn < MN) && (k < khi);
      if (ok[i])
        raw[i] = *reinterpret_cast<const U128*>(KMAJ ? p + mn * ld + k : p + k * ld + mn);
      else
        raw[i] = U128{{0, 0, 0, 0}};
    }
  }

  template <class PRE>
  __device__ __forceinline__ void store(bf16* lds, int64_t mn0, int64_t k0, int tid,
                                        const PRE& pre) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NTHR;
      if (PRE::kActive && ok[i]) {
        bf16* e = reinterpret_cast<bf16*>(&raw[i]);
        int64_t mn, k;
        if (KMAJ) {
          mn = mn0 + v / Geo::G;
          k = k0 + (v % Geo::G) * 8;
        } else {
          k = k0 + v / (ROWS / 8);
          mn = mn0 + (v % (ROWS / 8)) * 8;
        }
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = static_cast<float>(e[j]);
        pre.template vec<KMAJ, 8>(f, mn, k);
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = static_cast<bf16>(f[j]);
      }
      int off;
      if (KMAJ)
        off = Geo::kmaj_off(v / Geo::G, v % Geo::G);
      else
        off = (v / (ROWS / 8)) * Geo::PITCH + (v % (ROWS / 8)) * 8;
      *reinterpret_cast<U128*>(lds + off) = raw[i];
    }
  }
};

// Zero page for tile slots outside the matrix: lanes whose slot lies past
// M, N or K copy zeros from here, so ragged K tails contribute nothing.
static __device__ __attribute__((aligned(256))) uint32_t g_zero_page[256];

// Direct global->LDS stage loader (gfx950 global_load_lds, 16 bytes per
// lane): one wavefront instruction fills a contiguous 1 KiB of LDS, lane l
// writing bytes 16l .. 16l+15. Each lane therefore fetches the global
// element that belongs at its LDS slot (undoing the XOR swizzle of K-major
// tiles); slots in the row padding of MN-major tiles, or past the tile, are
// masked off. The data never passes through VGPRs and no ds_write is
// issued, so the LDS fill overlaps the MFMAs of the current stage.
template <int ROWS, int BK, bool KMAJ>
struct DirectLoader {
  using Geo = TileGeom<ROWS, BK, KMAJ>;
  static constexpr int BYTES = Geo::ELEMS * 2;
  static constexpr int CHUNKS = (BYTES + 1023) / 1024;
  static constexpr int NJ = (CHUNKS + 3) / 4;  // instructions per loading wavefront and stage

  // Streaming form: the byte offset of each of this lane's slots from the
  // tile's first element (row / column mn0 and k0 of the operand) is computed
  // once, so a stage fill costs one 64-bit add and one M0 update per
  // instruction; ~0u marks a slot with nothing to load (MN-major row
  // padding, or past the tile). Only for stages that lie inside K; rows or
  // columns past MN read the last one instead (the products of those never
  // reach a stored output).
  uint32_t off[NJ];
  __device__ __forceinline__ void init(int64_t ld, int64_t mn0, int64_t MN, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int o = (wave + 4 * q) * 1024 + lane * 16;
      if (KMAJ) {
        const int r = o / (BK * 2), pg = (o % (BK * 2)) / 16;
        const int g = pg ^ ((r / Geo::RPS) & (Geo::G - 1));
        const int64_t mn = min(mn0 + r, MN - 1);
        off[q] = o < BYTES ? (uint32_t)(((mn - mn0) * ld + g * 8) * 2) : ~0u;
      } else {
        const int r = o / (Geo::PITCH * 2), cb = o % (Geo::PITCH * 2);
        const int64_t mn = min(mn0 + cb / 2, MN - 8);
        off[q] = (o < BYTES && cb < ROWS * 2) ? (uint32_t)((r * ld + (mn - mn0)) * 2) : ~0u;
      }
    }
  }
  // tile = the operand at (mn0, k0): p + mn0 * ld + k0 (K-major) or
  // p + k0 * ld + mn0 (MN-major)
  __device__ __forceinline__ void issue_fast(const bf16* tile, bf16* lds, int wave) const {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int c = wave + 4 * q;
      if (c < CHUNKS && off[q] != ~0u) lds_fill16(tile, off[q], lds_addr(lds) + c * 1024);
    }
  }
  // `nw` loading wavefronts take the chunks wave, wave + nw, ...
  __device__ __forceinline__ static void issue(const bf16* __restrict__ p, int64_t ld, int64_t mn0,
                                               int64_t MN, int64_t k0, int64_t khi, bf16* lds,
                                               int wave, int lane, int nw = 4) {
#pragma unroll
    for (int c = wave; c < CHUNKS; c += nw) {
      const int o = c * 1024 + lane * 16;  // byte offset of this lane's slot
      int64_t mn, k;
      bool slot = o < BYTES;
      if (KMAJ) {
        const int r = o / (BK * 2), pg = (o % (BK * 2)) / 16;
        const int g = pg ^ ((r / Geo::RPS) & (Geo::G - 1));
        mn = mn0 + r;
        k = k0 + g * 8;
      } else {
        const int r = o / (Geo::PITCH * 2), cb = o % (Geo::PITCH * 2);
        slot = slot && cb < ROWS * 2;
        k = k0 + r;
        mn = mn0 + cb / 2;
      }
      const bool ok = (mn < MN) && (k < khi);
      const bf16* src = ok ? (KMAJ ? p + mn * ld + k : p + k * ld + mn)
                           : reinterpret_cast<const bf16*>(g_zero_page) + (lane & 15) * 8;
      if (slot) lds_fill16(src, lds_addr(lds) + c * 1024);
    }
  }
};

// Fragment of 32 operand rows starting at `row0` for the 16-wide
// contraction slice `ks` (lane l: row row0 + l%32, slots 8*(l/32) .. +7).
template <int ROWS, int BK, bool KMAJ>
__device__ __forceinline__ void read_frag(Frag<bf16>& f, const bf16* lds, int row0, int ks,
                                          int lane) {
  using Geo = TileGeom<ROWS, BK, KMAJ>;
  if (KMAJ) {
    const int r = row0 + (lane & 31);
    const int g = (lane >> 5) + 2 * ks;
    f.v = *reinterpret_cast<const bf16x8*>(lds + Geo::kmaj_off(r, g));
  } else {
    const int g16 = lane >> 4, L = lane & 15;
    const int k = ks * 16 + (g16 >> 1) * 8 + (L >> 2);
    const int m = row0 + (g16 & 1) * 16 + (L & 3) * 4;
    const bf16* p0 = lds + k * Geo::PITCH + m;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * Geo::PITCH));
    union {
      struct { v4i16 a, b; } s;
      bf16x8 v;
    } u;
    u.s.a = lo;
    u.s.b = hi;
    f.v = u.v;
  }
}

// ---------------------------------------------------------------- fp8 mode
// An fp8 operand tile is stored exactly like a bf16 K-major tile with BK
// 2-byte units per row: a 128-byte row holds 128 codes. One
// v_mfma_f32_32x32x64_f8f6f4 consumes a 64-wide contraction slice; lane l
// supplies 32 codes of row l % 32, bytes 32*(l/32) .. +31 of the slice. The
// instruction sums over all 64 slots, so any fixed assignment of lane bytes
// to contraction slots is correct as long as A and B use the same one.
typedef int i32x8 __attribute__((ext_vector_type(8)));
struct Frag8 {
  i32x8 v;
};

template <int ROWS, int BK>
__device__ __forceinline__ void read_frag8(Frag8& f, const bf16* lds, int row0, int ks, int lane) {
  using Geo = TileGeom<ROWS, BK, true>;
  const int r = row0 + (lane & 31);
  const int g = 4 * ks + 2 * (lane >> 5);
  const U128 lo = *reinterpret_cast<const U128*>(lds + Geo::kmaj_off(r, g));
  const U128 hi = *reinterpret_cast<const U128*>(lds + Geo::kmaj_off(r, g + 1));
  f.v = i32x8{(int)lo.w[0], (int)lo.w[1], (int)lo.w[2], (int)lo.w[3],
              (int)hi.w[0], (int)hi.w[1], (int)hi.w[2], (int)hi.w[3]};
}

// MODE 0: bf16 operands. MODE 1: e4m3 x e4m3. MODE 2: e5m2 (A) x e4m3 (B).
template <int MODE>
__device__ __forceinline__ void mfma8(f32x16& acc, const Frag8& a, const Frag8& b) {
  constexpr int FA = MODE == 2 ? 1 : 0;  // operand format codes: 0 e4m3, 1 e5m2
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, acc, FA, 0, 0, 0, 0, 0);
}

// The same with the B fragment first (the K-major kernel's C^T accumulator
// layout): the operand formats swap places.
template <int MODE>
__device__ __forceinline__ void mfma8_bt(f32x16& acc, const Frag8& b, const Frag8& a) {
  constexpr int FA = MODE == 2 ? 1 : 0;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b.v, a.v, acc, 0, FA, 0, 0, 0, 0);
}

// Dequantisation of an fp8 product. NoDeq: bf16 products. Deq8: in segment
// i of the M or N index (axis 0 or 1; at most 3 segments) the code sums are
// multiplied by f_i = 1 / (s_a,i * s_b,i), s = fmax / amax (1 if amax is 0
// or not finite). Scales that change along K are handled by the caller, one
// product per K segment (rescaling the accumulators inside the main loop
// would move them out of the accumulation registers).
struct NoDeq {
  static constexpr bool kOn = false;
  static constexpr bool kKseg = false;
};
// Aux type of an epilogue that reads no operand besides the accumulators.
struct NoAux {};

// Epilogues with kAmax also return max |stored value| per store (store4m,
// store4am); the block's maximum, rounded as stored (amax_of), is merged
// into *ep.amax with one integer atomic max (non-negative floats order like
// their bits) when that pointer is set.
template <class EP, class = void>
struct EpAmax : std::false_type {};
template <class EP>
struct EpAmax<EP, std::void_t<decltype(EP::kAmax)>> : std::integral_constant<bool, EP::kAmax> {};

// Epilogues with kStage32 stage 32 rows per pass at any width (the ReLU²
// ones: with 8-row passes their values stay live across more passes and
// spill).
template <class EP, class = void>
struct EpStage32 : std::false_type {};
template <class EP>
struct EpStage32<EP, std::void_t<decltype(EP::kStage32)>>
    : std::integral_constant<bool, EP::kStage32> {};

template <class EP>
__device__ __forceinline__ void amax_merge(const EP& ep, float mx) {
  if (ep.amax == nullptr) return;  // uniform over the block
  __shared__ float red[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = red[0];
    for (int q = 1; q < (int)(blockDim.x >> 6); ++q) v = fmaxf(v, red[q]);
    v = ep.amax_of(v);
    if (v > 0.0f) atomicMax(ep.amax, __float_as_uint(v));
  }
}
struct Deq8 {
  static constexpr bool kOn = true;
  static constexpr bool kKseg = false;
  const uint32_t* amax;
  int axis, nseg;  // axis 0: segments of M, 1: of N (Deq8K: of K, in codes)
  int64_t end[2];
  int sa[3], sb[3];
  float fa, fb;
  __device__ __forceinline__ int seg(int64_t i) const {
    return (nseg > 1 && i >= end[0]) + (nseg > 2 && i >= end[1]);
  }
};
// fp8 scales cut along the contraction (the K-major kernel only).
struct Deq8K : Deq8 {
  static constexpr bool kKseg = true;
};

// Scheduling groups for a main-loop slice: NR times (n MFMAs, one DS
// read), n = MP or MP + 1 so that the MFMAs spread evenly over the reads.
template <int R, int NR, int MP, int REM>
__device__ __forceinline__ void interleave_mfma_ds() {
  if constexpr (R < NR) {
    constexpr int n = MP + (R < REM ? 1 : 0);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x008, n, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                       // DS read
    interleave_mfma_ds<R + 1, NR, MP, REM>();
  }
}

// NW = 4: wavefronts in a 2 x 2 grid, one per SIMD. NW = 8 (bf16): a 4 x 2
// grid of (BM/4) x (BN/2) wavefront tiles, two wavefronts per SIMD, so one's
// LDS reads and waits overlap the other's MFMAs (half the accumulators per
// wavefront, more fragment reads per MFMA).
template <int BM, int BN, int BK, bool AK, bool BKM, int MODE, class PA, class PB, class EP,
          class DQ, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_bf16_kernel(
    const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, int64_t kchunk, int tiles_m, int tiles_n, PA pa, PB pb, EP ep_in,
    DQ dq, int64_t bsA, int64_t bsB) {
  static_assert(!PA::kActive && !PB::kActive, "direct LDS loads take operands as stored");
  constexpr bool F8 = MODE != 0;
  static_assert(!F8 || (AK && BKM), "fp8 products take K-major operands");
  static_assert(F8 == DQ::kOn, "fp8 products need a dequantisation");
  static_assert(NW == 4 || (NW == 8 && !F8), "8 wavefronts: bf16 products");
  using GA = TileGeom<BM, BK, AK>;
  using GB = TileGeom<BN, BK, BKM>;
  constexpr int WGM = NW / 2;            // wavefront rows of the block grid
  constexpr int WM = BM / WGM;           // wavefront tile rows
  constexpr int TM = WM / 32, TN = BN / 64;
  static_assert(TM >= 1 && WM % 32 == 0, "wavefront tile rows");
  constexpr int WN = BN / 2;
  constexpr int SP = WN + 4;  // epilogue staging row pitch (floats)
  constexpr int MAIN_BYTES = 2 * (GA::ELEMS + GB::ELEMS) * 2;
  constexpr int STAGE_BYTES = NW * 32 * SP * 4;
  __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > STAGE_BYTES ? MAIN_BYTES : STAGE_BYTES];
  bf16 (*As)[GA::ELEMS] = reinterpret_cast<bf16 (*)[GA::ELEMS]>(smem);
  bf16 (*Bs)[GB::ELEMS] = reinterpret_cast<bf16 (*)[GB::ELEMS]>(smem + 2 * GA::ELEMS * 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware, grouped tile order. The linear id runs over (split, tile),
  // split-major; consecutive ids are dealt to the 8 XCDs in turn, so the id
  // is remapped to give each XCD a contiguous range: its co-resident
  // workgroups then share one K range and neighbouring tiles in its L2. The
  // grid is padded to a multiple of 8; the padding workgroups exit here.
  const int ntiles = tiles_m * tiles_n;
  const int nwork = ntiles * (K > 0 && kchunk > 0 ? (int)((K + kchunk - 1) / kchunk) : 1);
  int pid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (pid >= nwork) return;
  const int split = pid / ntiles;
  pid -= split * ntiles;
  // batched products: gridDim.y independent problems, operands bsA / bsB
  // elements apart, the epilogue's own stride for C
  A += (int64_t)blockIdx.y * bsA;
  B += (int64_t)blockIdx.y * bsB;
  // split-K products write per-split partials
  const EP ep = ep_in.at_split(split).at_batch((int)blockIdx.y);
  constexpr int GM = 8;
  const int group = pid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % (GM * tiles_n)) % gsize;
  const int tn = (pid % (GM * tiles_n)) / gsize;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t k_lo = (int64_t)split * kchunk;
  const int64_t k_hi = min(K, k_lo + kchunk);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // fp8: dequantisation factor of each segment
  float fdq[3] = {1.0f, 1.0f, 1.0f};
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (i < dq.nseg)
        fdq[i] = 1.0f / (fp8_scale(dq.amax[dq.sa[i]], dq.fa) * fp8_scale(dq.amax[dq.sb[i]], dq.fb));
  }

  const int64_t nk = (k_hi - k_lo + BK - 1) / BK;
  // When both operands are K-major they stream straight into LDS; otherwise
  // both go through registers and are stored after the stage's MFMAs
  // (mixing the two fills measured slower than either).
  constexpr bool kDirect = AK && BKM;
  using DA = DirectLoader<BM, BK, AK>;
  using DB = DirectLoader<BN, BK, BKM>;
  Loader<BM, BK, AK, 64 * NW> ra;
  Loader<BN, BK, BKM, 64 * NW> rb;
  auto fetch = [&](int64_t k0, int buf) {
    if constexpr (kDirect) {
      DA::issue(A, lda, m0, M, k0, k_hi, As[buf], wave, lane, NW);
      DB::issue(B, ldb, n0, N, k0, k_hi, Bs[buf], wave, lane, NW);
    } else {
      ra.load(A, lda, m0, M, k0, k_hi, tid);
      rb.load(B, ldb, n0, N, k0, k_hi, tid);
    }
  };
  auto place = [&](int64_t k0, int buf) {
    if constexpr (!kDirect) {
      ra.store(As[buf], m0, k0, tid, pa);
      rb.store(Bs[buf], n0, k0, tid, pb);
    }
  };
  if (nk > 0) {
    fetch(k_lo, 0);
    place(k_lo, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's LDS fills landed
  __syncthreads();
  // Fragments of the next 16-wide k-slice are read into a second register
  // set before the MFMAs of the current slice are issued, so LDS latency
  // overlaps matrix work; the next stage streams in meanwhile.
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const int64_t kn = k_lo + (kt + 1) * BK;
    if (more) fetch(kn, cur ^ 1);
    if constexpr (F8) {
      // 64-wide contraction slices. A 32-code fragment takes 8 VGPRs, so fragments are not double-
      // buffered wholesale (that spills beside 256 accumulator registers):
      // the B fragments of the next slice and the A fragment of the next
      // row are read while the current row's MFMAs run.
      constexpr int KS = BK / 32;
      Frag8 b[2][TN], a[2];
#pragma unroll
      for (int j = 0; j < TN; ++j) read_frag8<BN, BK>(b[0][j], Bs[cur], wn * (BN / 2) + j * 32, 0, lane);
      read_frag8<BM, BK>(a[0], As[cur], wm * WM, 0, lane);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int p = ks & 1;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int q = i & 1;  // TM is even: row i of every slice uses a[i & 1]
          if (i + 1 < TM) {
            read_frag8<BM, BK>(a[q ^ 1], As[cur], wm * WM + (i + 1) * 32, ks, lane);
          } else if (ks + 1 < KS) {
            read_frag8<BM, BK>(a[q ^ 1], As[cur], wm * WM, ks + 1, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              read_frag8<BN, BK>(b[p ^ 1][j], Bs[cur], wn * (BN / 2) + j * 32, ks + 1, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < TN; ++j) mfma8<MODE>(acc[i][j], a[q], b[p][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // Slice 0 is read in the order its MFMAs consume it (A row 0, the B
      // columns, then the other A rows), one read at a time, so the first
      // MFMAs wait for two reads, not eight; the reads of slice ks + 1 are
      // interleaved with the MFMAs of slice ks.
      constexpr int KS = BK / 16;
      constexpr int NR = TM * (AK ? 1 : 2) + TN * (BKM ? 1 : 2);  // DS reads per slice
      constexpr int NM = TM * TN;
      Frag<bf16> a[2][TM], b[2][TN];
      auto read_slice = [&](int q, int ks, auto ordered) {
        read_frag<BM, BK, AK>(a[q][0], As[cur], wm * WM, ks, lane);
        if constexpr (decltype(ordered)::value) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          read_frag<BN, BK, BKM>(b[q][j], Bs[cur], wn * (BN / 2) + j * 32, ks, lane);
          if constexpr (decltype(ordered)::value) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 1; i < TM; ++i) {
          read_frag<BM, BK, AK>(a[q][i], As[cur], wm * WM + i * 32, ks, lane);
          if constexpr (decltype(ordered)::value) __builtin_amdgcn_sched_barrier(0);
        }
      };
      read_slice(0, 0, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int p = ks & 1;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) mfma(acc[i][j], a[p][i], b[p][j]);
        if (ks + 1 < KS) {
          read_slice(p ^ 1, ks + 1, std::false_type{});
          interleave_mfma_ds<0, NR, NM / NR, NM % NR>();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) place(kn, cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): next stage's direct fills landed
    __syncthreads();
  }

  const int64_t mw = m0 + wm * WM, nw = n0 + wn * WN;
  // Epilogue, one 32-row slab of the wavefront tile at a time: transform
  // the accumulators in their MFMA layout, stage the slab in LDS as fp32,
  // then write it back with 4-column vectors; all LDS reads of a slab are
  // issued before its first global store.
  // Epilogues that read another operand (residual, activation, old value)
  // load a whole slab of it at a time, a slab ahead where the registers
  // allow (two slab buffers of at most 64 VGPRs), else right after the
  // current slab's values are stored: the epilogue's time goes to the
  // latency of these loads, and a wavefront has only a few of them in
  // flight otherwise.
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * SP;
  constexpr bool kAux = !std::is_same<typename EP::Aux, NoAux>::value;
  constexpr int NVS = 32 * WN / 4 / 64;  // 4-column vectors per lane per slab
  constexpr int NCH = 2, CV = NVS / NCH;  // staged values are read in half slabs
  static_assert(NVS % NCH == 0, "value chunks must tile the slab");
  using AuxT = typename EP::Aux;
  constexpr int AUXR = kAux ? (int)(sizeof(AuxT) / 4) : 0;  // VGPRs per aux vector
  constexpr int NB = (kAux && NW == 4 && 2 * NVS * AUXR <= 64 && TM > 1) ? 2 : 1;
  // A tile wholly inside C takes the branch-free form: every 4-column vector
  // is whole and in range (per-vector range checks put each aux load on its
  // own branch, and the loads then issue one at a time).
  float amx = 0.0f;  // max |stored value| of this thread (kAmax epilogues)
  auto epilogue = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    auto in_range = [&](int64_t m, int64_t n) { return FULL || (m < M && n < N); };
    auto count = [&](int64_t n) { return FULL ? 4 : (int)min<int64_t>(4, N - n); };
    AuxT ax[kAux ? NB : 1][kAux ? NVS : 1];
    auto load_aux = [&](int i, AuxT* dst) {
#pragma unroll
      for (int t = 0; t < NVS; ++t) {
        const int v = lane + 64 * t;
        const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
        const int64_t m = mw + i * 32 + r, n = nw + c4;
        if (in_range(m, n)) dst[t] = ep.aux(m, n, count(n));
      }
    };
    if constexpr (kAux) load_aux(0, ax[0]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (kAux && NB == 2)
        if (i + 1 < TM) load_aux(i + 1, ax[(i + 1) % NB]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = acc_row(e, lane);
        const int64_t m = mw + i * 32 + r;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t n = nw + j * 32 + (lane & 31);
          float x = acc[i][j][e];
          if constexpr (F8) x *= fdq[dq.axis == 0 ? dq.seg(m) : dq.seg(n)];
          stage[r * SP + j * 32 + (lane & 31)] = ep.value(m, n, x);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staged slab visible to the wavefront
      __builtin_amdgcn_wave_barrier();
      if constexpr (kAux) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          f32x4 val[CV];
#pragma unroll
          for (int t = 0; t < CV; ++t) {
            const int v = lane + 64 * (c * CV + t);
            const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
            val[t] = *reinterpret_cast<const f32x4*>(stage + r * SP + c4);
          }
#pragma unroll
          for (int t = 0; t < CV; ++t) {
            const int v = lane + 64 * (c * CV + t);
            const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
            const int64_t m = mw + i * 32 + r, n = nw + c4;
            if (in_range(m, n)) {
              if constexpr (EpAmax<EP>::value)
                amx = fmaxf(amx, ep.store4am(m, n, val[t], count(n), ax[i % NB][c * CV + t]));
              else
                ep.store4a(m, n, val[t], count(n), ax[i % NB][c * CV + t]);
            }
          }
        }
        if constexpr (NB == 1)
          if (i + 1 < TM) load_aux(i + 1, ax[0]);
      } else {
        f32x4 val[NVS];
#pragma unroll
        for (int t = 0; t < NVS; ++t) {
          const int v = lane + 64 * t;
          const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
          val[t] = *reinterpret_cast<const f32x4*>(stage + r * SP + c4);
        }
#pragma unroll
        for (int t = 0; t < NVS; ++t) {
          const int v = lane + 64 * t;
          const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
          const int64_t m = mw + i * 32 + r, n = nw + c4;
          if (in_range(m, n)) {
            if constexpr (EpAmax<EP>::value)
              amx = fmaxf(amx, ep.store4m(m, n, val[t], count(n)));
            else
              ep.store4(m, n, val[t], count(n));
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  };
  if (m0 + BM <= M && n0 + BN <= N)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
  if constexpr (EpAmax<EP>::value) amax_merge(ep, amx);
}


// ---------------------------------------------------------------- K-major bf16 products
// Both operands K-major, bf16, K and the K chunk multiples of 64: 256-row
// tiles, 8 wavefronts in a 4 x 2 grid (wavefront tile 64 x BN/2), two LDS
// stages of 64-deep slabs filled straight from global memory.
//
// Schedule of one stage (four 16-wide slices). The fragments of slice s + 1
// are read while the MFMAs of slice s run. Before the last slice every
// wavefront waits for its own fills of the next stage and its own reads of
// this stage, then the workgroup synchronises: the next stage is now
// readable and this stage's buffer is free, so the fills of the stage after
// next are issued into it at once, and the last slice's MFMAs (whose
// fragments are already in registers) overlap the reads of the next
// stage's first slice. The barrier thus falls where every wavefront still
// has a whole slice of MFMAs queued, not at a point where all of them would
// first have to read LDS.
//
// The MFMA takes the B fragment as its first operand, so an accumulator
// block holds C^T: lane l owns row m = l % 32 and the four consecutive
// columns n = 8 (e / 4) + 4 (l / 32) + e % 4, e = 4g .. 4g + 3. The epilogue
// stages them with one 16-byte LDS write per group.
template <int ROWS>
struct KmajFill {
  static constexpr int CHUNKS = ROWS * 128 / 1024;  // 1 KiB LDS chunks of a stage
  static constexpr int NJ = CHUNKS / 8;             // per wavefront (8 wavefronts)
  static_assert(CHUNKS % 8 == 0, "whole chunks per wavefront");
  uint32_t off[NJ];
  // byte offset of each of this lane's slots from the tile origin (row mn0,
  // column k0); rows past MN read row MN - 1 (their products are never stored)
  __device__ __forceinline__ void init(int64_t ld, int64_t mn0, int64_t MN, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int o = (wave + 8 * q) * 1024 + lane * 16;
      const int r = o / 128, pg = (o % 128) / 16;
      const int g = pg ^ ((r / 2) & 7);
      const int64_t mn = min(mn0 + r, MN - 1);
      off[q] = (uint32_t)(((mn - mn0) * ld + g * 8) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16* tile, uint32_t lds, int wave) const {
#pragma unroll
    for (int q = 0; q < NJ; ++q) lds_fill16(tile, off[q], lds + (wave + 8 * q) * 1024);
  }
};

// Token-major (MN-major) stage of 64 contraction rows for the same kernel
// (TNL): LDS row k holds the ROWS output-index elements of contraction row
// k0 + k, with a pitch of ROWS + 32 elements, so the four rows a transposing
// fragment read touches start 64 bytes apart in the bank space and the
// gfx950 ds_read_b64_tr_b16 reads are conflict-free (see read_frag). A 1 KiB
// fill chunk runs across row ends; its lanes that land in a row's padding
// load that row's first 16 bytes again (never read back), so every lane of a
// fill takes part and no lane mask is needed. Columns past MN read the last
// 8 (their products are never stored).
template <int ROWS>
struct TnFill {
  static constexpr int PITCH = ROWS + 32;
  static constexpr int BYTES = 64 * PITCH * 2;
  static constexpr int CHUNKS = BYTES / 1024;
  static constexpr int NJ = (CHUNKS + 7) / 8;  // per wavefront (8 wavefronts; the last may idle)
  static_assert(BYTES % 1024 == 0, "whole chunks per stage");
  uint32_t off[NJ];
  // byte offset of each of this lane's slots from the tile origin (contraction
  // row k0, column mn0)
  __device__ __forceinline__ void init(int64_t ld, int64_t mn0, int64_t MN, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
      const int o = (wave + 8 * q) * 1024 + lane * 16;
      const int r = o / (PITCH * 2), cb = o % (PITCH * 2);
      const int col = cb < ROWS * 2 ? cb / 2 : 0;
      const int64_t mn = min(mn0 + col, MN - 8);
      off[q] = (uint32_t)(((int64_t)r * ld + (mn - mn0)) * 2);
    }
  }
  __device__ __forceinline__ void issue(const bf16* tile, uint32_t lds, int wave) const {
#pragma unroll
    for (int q = 0; q < NJ; ++q)
      if (wave + 8 * q < CHUNKS) lds_fill16(tile, off[q], lds + (wave + 8 * q) * 1024);
  }
};

//
// fp8 mode (MODE 1: e4m3 x e4m3, 2: e5m2 x e4m3; DQ = Deq8): the operands
// are codes handled as 2-byte units (K, the leading dimensions and the K
// chunk in units), so tiles, fills and LDS layout are unchanged; a 64-unit
// stage holds 128 codes per row and is consumed by two 64-code slices of
// v_mfma_f32_32x32x64_f8f6f4 (a fragment: 32 codes of one row per lane, two
// 16-byte reads), and the epilogue dequantises by segment.
//
// TNL: both operands token-major instead (the weight gradients: A(m, k) at
// A[k * lda + m], B(n, k) at B[k * ldb + n]), bf16 only. The stages hold
// TnFill's padded row-major tiles and the fragments are read with the
// transposing LDS load (read_frag), which yields the same register layout,
// so the schedule and the epilogue are unchanged.
template <int BN, class EP, int MODE = 0, class DQ = NoDeq, bool TNL = false>
__global__ __launch_bounds__(512) void gemm_kmaj_kernel(
    const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, int64_t kchunk, int tiles_m, int tiles_n, EP ep_in, int64_t bsA,
    int64_t bsB, DQ dq = DQ{}) {
  constexpr bool F8 = MODE != 0;
  static_assert(F8 == DQ::kOn, "fp8 products need a dequantisation");
  static_assert(!(TNL && F8), "token-major operands: bf16 only");
  constexpr int BM = 256, NW = 8, KS = F8 ? 2 : 4;
  constexpr int WM = BM / 4, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  // elements per stage
  constexpr int AEL = TNL ? TnFill<BM>::BYTES / 2 : BM * 64;
  constexpr int BEL = TNL ? TnFill<BN>::BYTES / 2 : BN * 64;
  constexpr int SP = WN + 4;                   // epilogue staging row pitch (floats)
  // rows of a wavefront's tile staged per epilogue pass: 32, or 8 for bf16
  // tiles wider than 256 columns and fp8 tiles of 256 (the staging area stays
  // within the LDS, and the staged values and operand loads of a pass fit
  // beside the accumulators and, in fp8 mode, the dequantisation factors)
  constexpr int RS = (WN > 128 || (F8 && WN == 128)) && !EpStage32<EP>::value ? 8 : 32;
  constexpr int MAIN_BYTES = 2 * (AEL + BEL) * 2;
  constexpr int STAGE_BYTES = NW * RS * SP * 4;
  __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > STAGE_BYTES ? MAIN_BYTES : STAGE_BYTES];
  const bf16* As = reinterpret_cast<const bf16*>(smem);
  const bf16* Bs = reinterpret_cast<const bf16*>(smem + 2 * AEL * 2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hi = lane >> 5;

  // tile order as in gemm_bf16_kernel: split-major, XCD-contiguous, groups
  // of 8 tile rows
  const int ntiles = tiles_m * tiles_n;
  const int nwork = ntiles * (int)((K + kchunk - 1) / kchunk);
  int pid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (pid >= nwork) return;
  const int split = pid / ntiles;
  pid -= split * ntiles;
  A += (int64_t)blockIdx.y * bsA;
  B += (int64_t)blockIdx.y * bsB;
  const EP ep = ep_in.at_split(split).at_batch((int)blockIdx.y);
  constexpr int GM = 8;
  const int group = pid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % (GM * tiles_n)) % gsize;
  const int tn = (pid % (GM * tiles_n)) / gsize;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t k_lo = (int64_t)split * kchunk;
  const int nk = (int)((min(K, k_lo + kchunk) - k_lo) / 64);

  std::conditional_t<TNL, TnFill<BM>, KmajFill<BM>> fa;
  std::conditional_t<TNL, TnFill<BN>, KmajFill<BN>> fb;
  fa.init(lda, m0, M, wave, lane);
  fb.init(ldb, n0, N, wave, lane);
  const bf16* Ab = TNL ? A + k_lo * lda + m0 : A + m0 * lda + k_lo;
  const bf16* Bb = TNL ? B + k_lo * ldb + n0 : B + n0 * ldb + k_lo;
  const int64_t sta = TNL ? 64 * lda : 64, stb = TNL ? 64 * ldb : 64;  // per stage
  const uint32_t la = lds_addr(As), lb = lds_addr(Bs);
  auto fill = [&](int kt, int buf) {
    fa.issue(Ab + (int64_t)kt * sta, la + buf * AEL * 2, wave);
    fb.issue(Bb + (int64_t)kt * stb, lb + buf * BEL * 2, wave);
  };
  auto kswz = [](int r, int g) { return r * 64 + ((g ^ ((r >> 1) & 7)) << 3); };
  auto fragA = [&](Frag<bf16>& f, int buf, int i, int ks) {
    if constexpr (TNL)
      read_frag<BM, 64, false>(f, As + buf * AEL, wm * WM + i * 32, ks, lane);
    else
      f.v = *reinterpret_cast<const bf16x8*>(As + buf * AEL + kswz(wm * WM + i * 32 + r32, 2 * ks + hi));
  };
  auto fragB = [&](Frag<bf16>& f, int buf, int j, int ks) {
    if constexpr (TNL)
      read_frag<BN, 64, false>(f, Bs + buf * BEL, wn * WN + j * 32, ks, lane);
    else
      f.v = *reinterpret_cast<const bf16x8*>(Bs + buf * BEL + kswz(wn * WN + j * 32 + r32, 2 * ks + hi));
  };
  // fp8: 32 codes of row r for 64-code slice ks: granules 4 ks + 2 hi, + 1
  auto frag8 = [&](Frag8& f, const bf16* base, int r, int ks) {
    const U128 lo = *reinterpret_cast<const U128*>(base + kswz(r, 4 * ks + 2 * hi));
    const U128 up = *reinterpret_cast<const U128*>(base + kswz(r, 4 * ks + 2 * hi + 1));
    f.v = i32x8{(int)lo.w[0], (int)lo.w[1], (int)lo.w[2], (int)lo.w[3],
                (int)up.w[0], (int)up.w[1], (int)up.w[2], (int)up.w[3]};
  };
  float fdq[3] = {1.0f, 1.0f, 1.0f};
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (i < dq.nseg)
        fdq[i] = 1.0f / (fp8_scale(dq.amax[dq.sa[i]], dq.fa) * fp8_scale(dq.amax[dq.sb[i]], dq.fb));
  }
  auto fsel = [&](int i) { return i == 0 ? fdq[0] : (i == 1 ? fdq[1] : fdq[2]); };
  // fp8 scales along K (axis 2; segment ends on 128-code stages): the
  // accumulators hold the sum in units of the current segment's factor, are
  // multiplied by f_prev / f_next where a stage opens the next segment, and
  // the epilogue applies the factor of the last segment
  int kseg = 0;
  if constexpr (DQ::kKseg) kseg = dq.seg(k_lo * 2);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  if (nk > 0) {
    fill(0, 0);
    if (nk > 1) {
      fill(1, 1);
      // vmcnt(fills of one stage): this wavefront's fills of stage 0 landed
      // (token-major stages: the count differs between wavefronts, so all)
      if constexpr (TNL)
        __builtin_amdgcn_s_waitcnt(0x0f70);
      else
        __builtin_amdgcn_s_waitcnt(0x0f70 | (KmajFill<BM>::NJ + KmajFill<BN>::NJ));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);
    }
  }
  __syncthreads();
  if constexpr (F8) {
    // two 64-code slices per stage; the fragments of slice s + 1 (of this
    // stage, or the next stage's first) are read while slice s's MFMAs run
    Frag8 a[2][TM], b[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) frag8(a[0][i], As, wm * WM + i * 32 + r32, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) frag8(b[0][j], Bs, wn * WN + j * 32 + r32, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (DQ::kKseg && kt > 0) {
        const int sg = dq.seg((k_lo + (int64_t)kt * 64) * 2);
        if (sg != kseg) {
          const float rr = fsel(kseg) / fsel(sg);
          kseg = sg;
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[i][j][e] *= rr;
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int p = ks & 1;
        if (ks == KS - 1) {
          __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
          __syncthreads();
          if (kt + 2 < nk) fill(kt + 2, cur);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) mfma8_bt<MODE>(acc[i][j], b[p][j], a[p][i]);
        const int rb = ks + 1 < KS ? cur : cur ^ 1, rs = ks + 1 < KS ? ks + 1 : 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) frag8(a[p ^ 1][i], As + rb * AEL, wm * WM + i * 32 + r32, rs);
#pragma unroll
        for (int j = 0; j < TN; ++j) frag8(b[p ^ 1][j], Bs + rb * BEL, wn * WN + j * 32 + r32, rs);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    Frag<bf16> a[2][TM], b[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fragA(a[0][i], 0, i, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) fragB(b[0][j], 0, j, 0);
    // LDS read instructions per slice: one per fragment, two for transposing reads
    constexpr int NR = (TNL ? 2 : 1) * (TM + TN), NM = TM * TN;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int p = ks & 1;
        if (ks == KS - 1) {
          // wave priority: 1 while issuing a slice's MFMAs and fragment reads,
          // 0 in the wait / barrier / fill section, so a wavefront in its
          // MFMA burst wins issue over its SIMD partner (d12 +0.2%)
          __builtin_amdgcn_s_setprio(0);
          __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
          __syncthreads();
          if (kt + 2 < nk) fill(kt + 2, cur);
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(1);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[p][j].v, a[p][i].v, acc[i][j], 0, 0, 0);
        // the next slice: of this stage, or the next stage's first (after the
        // last stage these reads are stale and unused)
        const int rb = ks + 1 < KS ? cur : cur ^ 1, rs = ks + 1 < KS ? ks + 1 : 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) fragA(a[p ^ 1][i], rb, i, rs);
#pragma unroll
        for (int j = 0; j < TN; ++j) fragB(b[p ^ 1][j], rb, j, rs);
        interleave_mfma_ds<0, NR, NM / NR, NM % NR>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __syncthreads();                     // the stage buffers become the epilogue's staging area

  // Epilogue, one 32-row slab of the wavefront tile at a time (see
  // gemm_bf16_kernel): transform, stage in LDS as fp32, write back in
  // 4-column vectors; operand-reading epilogues load a slab of the operand
  // ahead of its stores.
  const int64_t mw = m0 + wm * WM, nw = n0 + wn * WN;
  float* stage = reinterpret_cast<float*>(smem) + wave * RS * SP;
  constexpr bool kAux = !std::is_same<typename EP::Aux, NoAux>::value;
  constexpr int NVS = RS * WN / 4 / 64;
  constexpr int NCH = RS == 32 ? 2 : NVS, CV = NVS / NCH;
  constexpr int NH = 32 / RS;  // staging passes per 32-row slab
  static_assert(NVS % NCH == 0 && RS * WN / 4 % 64 == 0, "value chunks must tile the slab");
  using AuxT = typename EP::Aux;
  float amx = 0.0f;  // max |stored value| of this thread (kAmax epilogues)
  auto epilogue = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    auto in_range = [&](int64_t m, int64_t n) { return FULL || (m < M && n < N); };
    auto count = [&](int64_t n) { return FULL ? 4 : (int)min<int64_t>(4, N - n); };
    AuxT ax[kAux ? NVS : 1];
    auto load_aux = [&](int row0) {  // the operand of the RS rows from row0 of the wave tile
#pragma unroll
      for (int t = 0; t < NVS; ++t) {
        const int v = lane + 64 * t;
        const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
        const int64_t m = mw + row0 + r, n = nw + c4;
        if (in_range(m, n)) ax[t] = ep.aux(m, n, count(n));
      }
    };
    if constexpr (kAux) load_aux(0);
#pragma unroll
    for (int ih = 0; ih < TM * NH; ++ih) {
      const int i = ih / NH, h = ih % NH;
      const int64_t m = mw + i * 32 + r32;
      const bool mine = NH == 1 || r32 / RS == h;  // this lane's row is staged in this pass
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = j * 32 + 8 * g + 4 * hi;
          f32x4 v;
          // fp8: one dequantisation factor per 4-column group (segment
          // bounds are multiples of 4)
          float f = 1.0f;
          if constexpr (DQ::kKseg)
            f = fsel(kseg);
          else if constexpr (F8)
            f = fdq[dq.axis == 0 ? dq.seg(m) : dq.seg(nw + nl)];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[t] = ep.value(m, nw + nl + t, F8 ? acc[i][j][4 * g + t] * f : acc[i][j][4 * g + t]);
          if (mine) *reinterpret_cast<f32x4*>(stage + (r32 % RS) * SP + nl) = v;
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staged slab visible to the wavefront
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        f32x4 val[CV];
#pragma unroll
        for (int t = 0; t < CV; ++t) {
          const int v = lane + 64 * (c * CV + t);
          const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
          val[t] = *reinterpret_cast<const f32x4*>(stage + r * SP + c4);
        }
#pragma unroll
        for (int t = 0; t < CV; ++t) {
          const int v = lane + 64 * (c * CV + t);
          const int r = v / (WN / 4), c4 = (v % (WN / 4)) * 4;
          const int64_t mm = mw + i * 32 + h * RS + r, n = nw + c4;
          if (in_range(mm, n)) {
            if constexpr (kAux) {
              if constexpr (EpAmax<EP>::value)
                amx = fmaxf(amx, ep.store4am(mm, n, val[t], count(n), ax[c * CV + t]));
              else
                ep.store4a(mm, n, val[t], count(n), ax[c * CV + t]);
            } else {
              if constexpr (EpAmax<EP>::value)
                amx = fmaxf(amx, ep.store4m(mm, n, val[t], count(n)));
              else
                ep.store4(mm, n, val[t], count(n));
            }
          }
        }
      }
      if constexpr (kAux)
        if (ih + 1 < TM * NH) load_aux((ih + 1) / NH * 32 + (ih + 1) % NH * RS);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  };
  if (m0 + BM <= M && n0 + BN <= N)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
  if constexpr (EpAmax<EP>::value) amax_merge(ep, amx);
}

}  // namespace gk
