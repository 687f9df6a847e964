// Block-scaled E4M3 GEMM for gfx950 (CDNA4 matrix cores).
//
// Pages: paperlayer.ai summary of arXiv 2608.27370v1, appendix C
// "生産学習の詳細", item "FP8実装pipeline" -- the forward, data-gradient and
// weight-gradient GEMMs of each linear layer run on blockwise E4M3 operands;
// arxiv-wiki summary, section "접근 방법" item (4) -- one scale per 1x128
// activation group and per 128x128 weight block.
//
// One kernel family computes
//     C[i, j] = sum_lb SA(i, lb) * SB(j, lb) * P_lb[i, j],
//     P_lb[i, j] = sum_{l in block lb} A[i, l] * B[j, l]      (E4M3 codes)
// with both operands contraction-contiguous ("NT"), which is the natural
// layout of all three GEMMs:
//     forward  C = Y  [M, N]: A = Xq   [M, K],  B = Wq  [N, K]   (SB per 128x128 block)
//     dgrad    C = dX [M, K]: A = dYq  [M, N],  B = WqT [K, N]   (SB per 128x128 block)
//     wgrad    C = dW [N, K]: A = dYqT [N, M],  B = XqT [K, M]   (SB per row)
//
// gfx950 design:
//   * operands stay E4M3 in HBM and LDS (one byte per element).  Each
//     workgroup stages a BM x 128 tile of A, a BN x 128 tile of B and their
//     per-row scales per scale block straight into LDS (global_load_lds, no
//     VGPR round trip), into one of several buffers: for large problems three,
//     so blocks lb+1 and lb+2 stream in while block lb is multiplied.  The
//     buffers are distinct LDS objects and the block loop is unrolled by the
//     buffer count.  Fills are waited for explicitly and synchronised with an
//     LDS-only barrier (a full __syncthreads() would drain every fill in
//     flight).  Rows are 128 bytes with the 16-byte chunks XOR-swizzled by
//     (row / 2) % 8, so fragment reads (ds_read_b128) are bank-conflict free;
//   * the block product of a sub-tile is formed in the matrix core from a zero
//     accumulator and folded into FP32 register accumulators with one FMA per
//     element and block (acc = fma(P_lb, SA*SB, acc)):
//       exact path (default): E4M3 codes are converted exactly to F16 in
//         registers and multiplied with v_mfma_f32_32x32x16_f16, eight per
//         32x32 sub-tile and block; the K slices of a block are read from LDS
//         one ahead of the multiply, and the first slice of the next block is
//         read while the last one is multiplied;
//       FP8 matrix-core path (opt-in): two v_mfma_f32_32x32x64_f8f6f4 per
//         32x32 sub-tile and block on the codes (twice the matrix rate, but
//         the hardware truncates small products inside groups of 8, see Prec);
//   * workgroups are renumbered so that each of the 8 XCDs (own L2) works on a
//     contiguous range of output tiles, grouped a few tile-rows at a time;
//   * the output tile leaves through LDS, so that every store instruction
//     writes whole 16-byte chunks of complete row segments.
#include "internal.h"
#include "fp8_codec.h"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

constexpr int BK = 128;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained; gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }
// The same with an lgkmcnt limit as well (63 leaves vmcnt unconstrained).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | (0x7 << 4) | ((lgkm & 0xF) << 8) | (((vm >> 4) & 3) << 14);
}

// PREC selects how the 128-term block product is formed:
//   PREC_F16: the E4M3 codes are converted exactly to F16 in registers
//     (v_cvt_scalef32_pk_f16_fp8 with scale 1; every E4M3 value is an F16
//     normal or zero) and multiplied with v_mfma_f32_32x32x16_f16.  The
//     matrix core adds the products of one instruction without intermediate
//     truncation, so the block partial carries only FP32 rounding (a few
//     2^-24 relative).
//   PREC_FP8: two v_mfma_f32_32x32x64_f8f6f4 per 32x32 sub-tile and block, on
//     the codes themselves.  On gfx950 the FP8 matrix instructions sum
//     products in groups of 8 after aligning them to the largest product of
//     the group and truncating 13 bits below it, so a block partial can be off
//     by up to about 7 * 2^-13 of the group's largest product when values
//     inside a group differ widely in magnitude.
enum Prec { PREC_F16 = 0, PREC_FP8 = 1 };

// Eight E4M3 codes (two dwords) -> one F16 MFMA operand, exact.
__device__ __forceinline__ v8h cvt8(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Tile-rows per group of the launch order.  Each XCD fetches, round by round,
// the A row panels and B column panels of the tiles it runs at once (its 4 MB
// L2 keeps nothing from one round for the next), so a round's r x c tiles
// cost r * BM + c * BN rows of operand: with 32 tiles per XCD that is least
// at 4 x 8 for 256 x 128 tiles and 8 x 8 for 128 x 128 tiles (two per CU).
template <int BM>
constexpr int group_rows() { return BM == 256 ? 4 : 8; }

// With split-K (S > 1) the grid holds S workgroups per tile: the S splits of a
// tile are consecutive logical units, so they usually share an XCD.  Returns
// the tile's index in the grouped order and sets its coordinates and this
// workgroup's split.
template <int GM, int S>
__device__ __forceinline__ int map_tile(int pid, int nblocks, int tilesM, int tilesN, int& tm, int& tn, int& split) {
  // Workgroup pid runs on XCD pid % 8; give each XCD a contiguous logical range.
  const int q = nblocks / 8, r = nblocks % 8;
  const int xcd = pid % 8, local = pid / 8;
  const int logical = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  split = logical % S;
  const int tile = logical / S;
  // Grouped order: GM tile-rows at a time, walking down columns.
  const int per_group = GM * tilesN;
  const int gid = tile / per_group;
  const int first_m = gid * GM;
  const int gm = min(tilesM - first_m, GM);
  const int in_group = tile - gid * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
  return tile;
}

// Split-K rendezvous, called by every thread once its split's FP32 partial
// tile is stored in the workspace.  The workgroup barrier makes every wave's
// stores happen before thread 0's count on the tile's counter, which is an
// agent-scope release (other XCDs have their own L2); the workgroup whose count
// completes the tile performs the matching acquire and returns true: it reads
// the other splits' partials and stores the tile.  It also puts the counter
// back to zero, so a workspace whose counters start at zero is left that way by
// every call.  One release per workgroup and one acquire per tile keep the
// cache maintenance these imply off the other workgroups' operand reuse; no
// workgroup ever waits for another, so the scheme needs no co-residency.
template <int S>
__device__ __forceinline__ bool split_arrive(unsigned* counter, int t, int* flag) {
  __syncthreads();
  if (t == 0) {
    const unsigned arrived = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = arrived == S - 1;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// The tile's value from its S partials, added in split order (split 0 +
// split 1 + ... + split S-1) into acc, which holds this workgroup's own
// partial (split `split`).  `first` is this lane's float of split 0 and
// `stride` the distance between splits; partial (mt, nt, q) of a lane is the
// float4 at ((mt * NT + nt) * 4 + q) * 256.  The loop over the splits is kept
// rolled so that one split's loads (16 registers per sub-tile) are live at a
// time.
template <int S, int MT, int NT>
__device__ __forceinline__ void add_partials(float (&acc)[MT][NT][16], const float* first, int64_t stride, int split) {
  float tot[MT][NT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v;
        if (split == 0)
          v = make_float4(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
        else
          v = *reinterpret_cast<const float4*>(first + ((mt * NT + nt) * 4 + q) * 256);
        tot[mt][nt][4 * q] = v.x; tot[mt][nt][4 * q + 1] = v.y;
        tot[mt][nt][4 * q + 2] = v.z; tot[mt][nt][4 * q + 3] = v.w;
      }
#pragma unroll 1
  for (int sp = 1; sp < S; ++sp) {
    const float* src = first + sp * stride;
    if (sp == split) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 16; ++e) tot[mt][nt][e] += acc[mt][nt][e];
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(src + ((mt * NT + nt) * 4 + q) * 256);
            tot[mt][nt][4 * q] += v.x; tot[mt][nt][4 * q + 1] += v.y;
            tot[mt][nt][4 * q + 2] += v.z; tot[mt][nt][4 * q + 3] += v.w;
          }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = tot[mt][nt][e];
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// releases global memory, which makes every wave wait for all of its
// outstanding global loads (vmcnt(0)) -- including the direct-to-LDS fills of
// blocks that are meant to stay in flight across the barrier.  Fills that must
// have landed are waited for explicitly (s_waitcnt vmcnt) before this call.
// The wave's own LDS reads are completed first (lgkmcnt(0)), so no fill
// issued after the barrier can overwrite data a read has not fetched yet; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte offset of 16-byte chunk `chunk` of tile row `row` in LDS.  gfx950
// serves a ds_read_b128 sixteen lanes at a time from 256 bytes of banks, so
// the sixteen rows a fragment read touches must land in sixteen distinct
// 16-byte bank slots: row parity picks the 128-byte half, and the chunk is
// XOR-ed with (row / 2) % 8 (measured conflict-free; XOR with row % 8 makes
// rows r and r + 8 collide, 4 extra cycles per read).
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_key(row)) << 4); }

__device__ __forceinline__ uint4 lds16(const uint8_t* tile, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(tile + swz(row, chunk));
}

// Direct-to-LDS copies (global_load_lds, saddr form): lane L copies 16 (or 4)
// bytes from base + voff to LDS address lds + 16 L (4 L).  They are issued from
// inline assembly on purpose: for the builtin, the compiler cannot tell which
// LDS buffer a fill targets and makes every later LDS read wait for all fills
// in flight (vmcnt(0)), which would serialise the multi-buffered pipeline.  The
// statements have no register outputs; every consumer of a fill waits for it
// explicitly (s_waitcnt vmcnt) and then synchronises the workgroup.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t)p;
}
__device__ __forceinline__ void dma_b128(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
               :: "s"(base), "v"(voff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, %0"
               :: "s"(base), "v"(voff), "s"(lds) : "memory", "m0");
}

// Direct-to-LDS staging.  A tile of ROWS rows x 128 bytes moves with ROWS/8
// wave instructions of 1 KB; lane L of instruction `blk` writes LDS bytes
// [16L, 16L+16) of its 1 KB, i.e. tile row r = 8 blk + L/8, slot L%8, which
// must hold global chunk (L%8) ^ swz_key(r) of that row.  The per-lane byte
// offsets are relative to the tile's first row and loop invariant (computed
// once; 32-bit, which holds for any row stride below 2^23 bytes whatever the
// operand's size); per scale block only the wave-uniform 64-bit base pointer
// moves, so each load is one instruction with no address arithmetic.  Rows
// past the last valid row are clamped to it; they only feed output rows that
// are never stored.
template <int ROWS, int NW>
struct TileStager {
  static constexpr int kLoads = ROWS / (8 * NW);   // instructions per wave
  static_assert(kLoads * 8 * NW == ROWS, "tile rows must split evenly over the waves");
  uint32_t off[kLoads];
  __device__ __forceinline__ void init(int64_t ld, int64_t r0, int64_t rmax, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int trow = 8 * (NW * u + wave) + (lane >> 3);   // row within the tile
      int64_t row = r0 + trow;
      row = row < rmax ? row : rmax;
      off[u] = (uint32_t)((row - r0) * ld) + (uint32_t)(((lane & 7) ^ swz_key(trow)) * 16);
    }
  }
  // base: G + r0 * ld + lb * 128 (wave-uniform); dst: the tile in LDS.
  __device__ __forceinline__ void issue(const uint8_t* base, uint8_t* dst, int wave) const {
    const uint32_t l0 = lds_addr(dst) + wave * 1024;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) dma_b128(base, off[u], l0 + NW * u * 1024);
  }
};

// N scale values SC[lb * ld + r0 + r] (indices clamped to rmax) into LDS with
// 4-byte direct loads, N/NW per wave (one instruction each).
template <int N, int NW>
struct ScaleStager {
  static constexpr int kPerWave = N / NW;
  static_assert(kPerWave <= 64, "one instruction per wave");
  uint32_t off;
  __device__ __forceinline__ void init(int64_t r0, int64_t rmax, int wave, int lane) {
    int64_t r = r0 + kPerWave * wave + (lane < kPerWave ? lane : 0);
    r = r < rmax ? r : rmax;
    off = (uint32_t)(r - r0) * 4u;   // relative to the tile's first row
  }
  // base: SC + lb * ld + r0 (wave-uniform).
  __device__ __forceinline__ void issue(const float* base, float* dst, int wave, int lane) const {
    const uint32_t l0 = lds_addr(dst + kPerWave * wave);
    if (lane < kPerWave) dma_b32(base, off, l0);
  }
};

// Epilogue through LDS.  Stored straight from the MFMA result registers, a
// wave store touches many rows with a few bytes each (the accumulator layout
// spreads a lane's values down a column).  Instead each wave writes a band of
// its output tile (BAND rows x WN columns) into a private LDS region, reads it
// back row-major and stores whole 16-byte chunks: one wave instruction then
// covers complete WN-column row segments (8 of them for BF16, 4 for FP32).
// The stage buffers hold the regions once every wave is past the main loop.
// The row stride is padded by 16 bytes to spread a band's rows over the banks.
// Two binary32 values -> packed BF16, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int OUT, int WN>
struct Band {
  static constexpr int ESZ = OUT == OUT_BF16 ? 2 : 4;
  static constexpr int RS = WN * ESZ + 16;      // row stride in LDS (bytes)
  static constexpr int CPR = WN * ESZ / 16;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per wave instruction
  static_assert(CPR * RPI == 64, "a band row splits evenly over the wave");
};

// This wave's region of REGION bytes: regions are packed into the stage
// buffers (BUF bytes each, NS of them) in wave order.
template <int REGION, int BUF, int NS, int NW>
__device__ __forceinline__ uint8_t* band_region(uint8_t* lds0, uint8_t* lds1, uint8_t* lds2, int wave) {
  constexpr int PER_BUF = BUF / REGION;
  static_assert(PER_BUF * NS >= NW, "epilogue regions must fit in the stage buffers");
  const int bi = wave / PER_BUF;
  return (bi == 0 ? lds0 : bi == 1 ? lds1 : lds2) + (wave % PER_BUF) * REGION;
}

// Read a band of ROWS rows back from `region` and store row r at output row
// row0 + r (rows at or past I are skipped), columns col0 .. col0 + WN - 1;
// OUT_F32_ACC adds the values already in C.
template <int OUT, int WN, int ROWS>
__device__ __forceinline__ void store_band(const uint8_t* region, int lane, void* Cout, int64_t ldc,
                                           int64_t row0, int64_t col0, int64_t I) {
  using Bd = Band<OUT, WN>;
  static_assert(ROWS % Bd::RPI == 0, "band rows split over the wave instructions");
  uint8_t* cbase = static_cast<uint8_t*>(Cout) + col0 * Bd::ESZ;
#pragma unroll
  for (int it = 0; it < ROWS / Bd::RPI; ++it) {
    const int r = it * Bd::RPI + lane / Bd::CPR, k = lane % Bd::CPR;
    const uint4 w = *reinterpret_cast<const uint4*>(region + r * Bd::RS + k * 16);
    const int64_t row = row0 + r;
    if (row >= I) continue;
    uint8_t* dst = cbase + row * ldc * Bd::ESZ + k * 16;
    if (OUT == OUT_F32_ACC) {
      const float4 old = *reinterpret_cast<const float4*>(dst);
      float4 o = *reinterpret_cast<const float4*>(&w);
      o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
      *reinterpret_cast<float4*>(dst) = o;
    } else {
      *reinterpret_cast<uint4*>(dst) = w;
    }
  }
}

template <int BM, int BN, int WM, int WN, int SB_MODE, int PREC, int NW, int NS>
struct Cfg {
  static constexpr int WGM = BM / WM, WGN = BN / WN;
  static_assert(WGM * WGN == NW, "one wave per WM x WN sub-tile");
  static_assert(NS == 2 || NS == 3, "double or triple buffering");
  // Vector-memory instructions one wave issues to stage one block.
  static constexpr int kVmemPerBlock =
      TileStager<BM, NW>::kLoads + TileStager<BN, NW>::kLoads + 1 + (SB_MODE == SB_ROWS ? 1 : 0);
  // Sub-tile edge: 32 on both paths (32x32x16 F16 and 32x32x64 FP8 MFMAs).
  static constexpr int T = 32;
  static constexpr int MT = WM / T, NT = WN / T;
  // Per-buffer LDS layout: A tile, B tile, BM row scales of A.  The BN row
  // scales of B (SB_ROWS) go to a ring of NS + 1 slots of their own
  // (kRing), so that a block's scales survive the refill of its stage buffer
  // and can be read after the block-end barrier.
  static constexpr int kSaOff = (BM + BN) * BK;
  static constexpr int kBufBytes = kSaOff + BM * 4;
  static constexpr int kRing = NS + 1;
};

// Exact path: E4M3 -> F16 in registers, v_mfma_f32_32x32x16_f16; one
// workgroup per output tile.
// Split-K (S > 1): workgroup `split` of a tile contracts over scale blocks
// [nLBtot * split / S, nLBtot * (split + 1) / S).  Without PLANES, `part`
// holds S FP32 partial tiles per output tile and `cnt` one arrival counter per
// output tile, and the last split to arrive stores the tile; with PLANES each
// split stores its FP32 partial into plane `split` of Cout ([S][I][ldc]) and a
// second kernel (add_planes_kernel) adds the planes.
template <int BM, int BN, int WM, int WN, int SB_MODE, int OUT, int NW, int NS, int S, bool PLANES>
__global__ __launch_bounds__(64 * NW, (NW == 4 && NS == 2) ? 2 : 1) void block_gemm_f16_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ SB, int64_t ldsb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN,
    float* __restrict__ part, unsigned* __restrict__ cnt) {
  using C = Cfg<BM, BN, WM, WN, SB_MODE, PREC_F16, NW, NS>;
  constexpr int MT = C::MT, NT = C::NT;
  // One distinct LDS object per pipeline stage (see the file comment).
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NS == 3 ? C::kBufBytes : 16];
  __shared__ __attribute__((aligned(16))) float sb_ring[SB_MODE == SB_ROWS ? C::kRing * BN : 4];
  __shared__ int split_flag;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int tm, tn, split;
  const int tile = map_tile<group_rows<BM>(), S>(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn, split);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int nLBtot = (int)(L / BK);
  const int lb0 = nLBtot * split / S;
  const int nLB = nLBtot * (split + 1) / S - lb0;   // this split's scale blocks
  // Lane l: row (l % 32) of a 32x32 sub-tile; half h = l / 32 holds K bytes
  // [64h, 64h + 64) of the block.  K slice c (0..3) is the 16 bytes at
  // 64h + 16c, one LDS read per fragment row; MFMA k (0, 1) of the slice takes
  // its 8 codes at 64h + 16c + 8k.  The MFMA is given the B fragment first, so
  // it produces the transposed sub-tile: lane l holds output row (l % 32) --
  // one A row, hence one A scale per lane -- and accumulator 4q + u holds
  // output column 8q + 4h + u.
  const int h = lane >> 5, rr = lane & 31;

  float acc[MT][NT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  TileStager<BM, NW> sta;
  TileStager<BN, NW> stb;
  ScaleStager<BM, NW> ssa;
  ScaleStager<BN, NW> ssb;
  sta.init(lda, i0, I - 1, wave, lane);
  stb.init(ldb, j0, j0 + BN - 1, wave, lane);
  ssa.init(i0, I - 1, wave, lane);
  ssb.init(j0, j0 + BN - 1, wave, lane);
  auto stage_all = [&](int lbl, uint8_t* buf) {
    const int64_t lb = lb0 + lbl;
    sta.issue(A + i0 * lda + lb * BK, buf, wave);
    stb.issue(B + j0 * ldb + lb * BK, buf + BM * BK, wave);
    ssa.issue(SA + lb * ldsa + i0, reinterpret_cast<float*>(buf + C::kSaOff), wave, lane);
    if (SB_MODE == SB_ROWS) ssb.issue(SB + lb * ldsb + j0, sb_ring + (lbl % C::kRing) * BN, wave, lane);
  };

  uint4 qa[2][MT], qb[2][NT];   // raw codes of two K slices (software pipeline)
  // Converted operands: two K slices with the deeper schedule below, else one.
  constexpr bool kAhead = NW == 8 && SB_MODE == SB_BLOCK;
  v8h fa[2][MT][2], fb[2][NT][2];
  v16f p[MT][NT];               // block products
  auto load_slice = [&](const uint8_t* buf, int c, int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) qa[slot][mt] = lds16(buf, wm * WM + mt * 32 + rr, 4 * h + c);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qb[slot][nt] = lds16(buf + BM * BK, wn * WN + nt * 32 + rr, 4 * h + c);
    // Only VALU and SALU work may be scheduled across this point: the reads
    // stay a slice ahead instead of sinking next to their first use.
    __builtin_amdgcn_sched_barrier(0x0006);
  };
  // Codes of slot `slot` -> converted operands of slot `fs`.
  auto convert = [&](int slot, int fs) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      fa[fs][mt][0] = cvt8(qa[slot][mt].x, qa[slot][mt].y);
      fa[fs][mt][1] = cvt8(qa[slot][mt].z, qa[slot][mt].w);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      fb[fs][nt][0] = cvt8(qb[slot][nt].x, qb[slot][nt].y);
      fb[fs][nt][1] = cvt8(qb[slot][nt].z, qb[slot][nt].w);
    }
  };
  auto multiply = [&](int fs) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          p[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[fs][nt][k], fa[fs][mt][k], p[mt][nt], 0, 0, 0);
  };

  // Block lb from `cur`.
  // Two schedules.  With 8 waves (two per SIMD) and block scales of B (the
  // forward and data-gradient GEMMs): on entry slice 0 is converted (operand
  // slot 0)
  // and the codes of slice 1 are read (code slot 1).  Each slice's MFMAs use
  // operands converted during the slice before, while the next slice is
  // converted and the one after it read, so a wave's MFMAs never wait for its
  // own conversions.  Slices 2 and 3 are multiplied before the block-end
  // barrier (they run while the wave waits there for the slowest wave); after
  // it `cur` is refilled with block lb + NS, slices 0 and 1 of block lb + 1 are
  // read from `nxt` and slice 0 is converted.
  // Otherwise one operand slot: slice 0 is read on entry, slices 1..3 are
  // read one ahead of the multiply, each converted just before it; with 8
  // waves slice 3 is multiplied before the barrier, with 4 after it, once
  // `cur` is refilled and slice 0 of block lb + 1 is read.  (The second slot
  // was measured: 2% faster on the forward and data-gradient GEMMs, 4% slower
  // on the 8-wave weight gradients, which then need 254 registers; the 4-wave
  // tiles, two workgroups per CU, spill with it.)
  // The block's scales are read into registers before `cur` can be refilled.
  auto step = [&](uint8_t* cur, const uint8_t* nxt, int lb) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p[mt][nt] = v16f{};
    if constexpr (kAhead) {
      load_slice(cur, 2, 0);
      convert(1, 1);
      multiply(0);
      load_slice(cur, 3, 1);
      convert(0, 0);
      multiply(1);
      convert(1, 1);
      multiply(0);
      multiply(1);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        load_slice(cur, c + 1, (c + 1) & 1);
        convert(c & 1, 0);
        multiply(0);
      }
      convert(1, 0);
      if (NW == 8) {
        multiply(0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float* lsa = reinterpret_cast<const float*>(cur + C::kSaOff);
    float sa[MT];                  // A scale of this lane's output row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa[mt] = lsa[wm * WM + mt * 32 + rr];
    const float sblk = (SB_MODE == SB_BLOCK) ? SB[(j0 / 128) * nLBtot + lb0 + lb] : 1.0f;
    if (NS == 3 && lb + 2 < nLB)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kVmemPerBlock));   // block lb+1 landed, lb+2 may fly
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    if (lb + NS < nLB) stage_all(lb + NS, cur);
    if constexpr (kAhead) {
      if (lb + 1 < nLB) {
        load_slice(nxt, 0, 0);
        load_slice(nxt, 1, 1);
        convert(0, 0);
      }
    } else {
      if (lb + 1 < nLB) load_slice(nxt, 0, 0);
      if (NW != 8) multiply(0);
    }
    float4 sbr[NT][4];             // SB_ROWS: B scales of output columns 8q + 4h + u
    const float* lsb = sb_ring + (lb % C::kRing) * BN;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sbr[nt][q] = (SB_MODE == SB_ROWS) ? *reinterpret_cast<const float4*>(lsb + wn * WN + nt * 32 + 8 * q + 4 * h)
                                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    // Rescale-accumulate: acc += P * SA(row) * SB.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float srow = (SB_MODE == SB_BLOCK) ? sa[mt] * sblk : sa[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float cs[4] = {sbr[nt][q].x, sbr[nt][q].y, sbr[nt][q].z, sbr[nt][q].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sc = (SB_MODE == SB_ROWS) ? srow * cs[u] : srow;
            acc[mt][nt][4 * q + u] = fmaf(p[mt][nt][4 * q + u], sc, acc[mt][nt][4 * q + u]);
          }
        }
    }
  };

  // Prologue: fill every buffer, wait for block 0, read its slice 0.
  const int pre = nLB < NS ? nLB : NS;
  stage_all(0, lds0);
  if (pre > 1) stage_all(1, lds1);
  if (NS == 3 && pre > 2) stage_all(2, lds2);
  if (NS == 3 && pre > 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::kVmemPerBlock));
  else if (pre > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kVmemPerBlock));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  load_slice(lds0, 0, 0);
  if (kAhead) {
    load_slice(lds0, 1, 1);
    convert(0, 0);
  }
  if (NS == 2) {
    for (int lb = 0; lb < nLB; lb += 2) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds0, lb + 1);
    }
  } else {
    for (int lb = 0; lb < nLB; lb += 3) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds2, lb + 1);
      if (lb + 2 < nLB) step(lds2, lds0, lb + 2);
    }
  }

  if (S > 1 && !PLANES) {
    // Split-K: store this split's partial tile lane-major (one 1 KB run per
    // wave instruction); the last split to arrive adds the S partials in split
    // order -- its own from registers -- and goes on to store the tile.
    constexpr int kWave = MT * NT * 16 * 64;    // floats per wave and split
    float* mine = part + ((int64_t)(tile * S + split) * NW + wave) * kWave + lane * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(mine + ((mt * NT + nt) * 4 + q) * 256) =
              make_float4(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
    if (!split_arrive<S>(cnt + tile, t, &split_flag)) return;
    add_partials<S, MT, NT>(acc, part + ((int64_t)tile * S * NW + wave) * kWave + lane * 4, NW * kWave, split);
  }

  // Epilogue, one 32-row band (sub-tile row mt) at a time through LDS.  Lane l
  // holds row (l % 32) of the band and, in accumulators 4q..4q+3 of sub-tile
  // nt, the four consecutive columns nt * 32 + 8q + 4h .. + 3.
  lds_barrier();
  {
    using Bd = Band<OUT, WN>;
    static_assert(!PLANES || (S > 1 && OUT == OUT_F32), "partial planes are FP32");
    // Small-grid split: this split's partial goes to plane `split` of the
    // workspace ([S][I][ldc] FP32); add_planes_kernel adds the planes.
    void* dst = PLANES ? static_cast<void*>(static_cast<float*>(Cout) + (int64_t)split * I * ldc) : Cout;
    uint8_t* region = band_region<32 * Bd::RS, C::kBufBytes, NS, NW>(lds0, lds1, lds2, wave);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* v = &acc[mt][nt][4 * q];
          uint8_t* p = region + rr * Bd::RS + (nt * 32 + 8 * q + 4 * h) * Bd::ESZ;
          if (OUT == OUT_BF16) {
            *reinterpret_cast<uint2*>(p) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
          } else {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      store_band<OUT, WN, 32>(region, lane, dst, ldc, i0 + wm * WM + mt * 32, j0 + wn * WN, I);
    }
  }
}

// Exact path, 128 x 128 tiles of 8 waves in two K groups.  Waves 0-3 and 4-7
// each cover the tile with 64 x 64 sub-tiles and contract one half of the
// scale blocks (the first and the second half) through double-buffered
// stages of their own; the second group's accumulators are then added to the
// first group's through LDS, one FP32 add per element in that fixed order, and
// the first group stores the tile.  For grids of about one 128 x 128 tile per
// CU this gives every SIMD two waves instead of one.  Both groups meet every
// workgroup barrier, so the number of scale blocks must be even.
template <int SB_MODE, int OUT>
__global__ __launch_bounds__(512, 1) void block_gemm_f16_kgroups_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ SB, int64_t ldsb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, NWG = 4, NS = 2;
  using C = Cfg<BM, BN, WM, WN, SB_MODE, PREC_F16, NWG, NS>;
  constexpr int MT = C::MT, NT = C::NT;
  // Stage buffers of group 0 and of group 1 (distinct LDS objects).
  __shared__ __attribute__((aligned(1024))) uint8_t g0s0[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t g0s1[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t g1s0[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t g1s1[C::kBufBytes];
  __shared__ __attribute__((aligned(16))) float sb_ring[2][SB_MODE == SB_ROWS ? C::kRing * BN : 4];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, lw = wave & 3;
  int tm, tn, split;
  map_tile<group_rows<BM>(), 1>(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn, split);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = lw / C::WGN, wn = lw % C::WGN;
  const int nLBtot = (int)(L / BK);
  const int nLB = nLBtot / 2;            // this group's scale blocks
  const int lb0 = grp * nLB;
  const int h = lane >> 5, rr = lane & 31;
  uint8_t* const lds0 = grp ? g1s0 : g0s0;
  uint8_t* const lds1 = grp ? g1s1 : g0s1;
  float* const ring = sb_ring[grp];

  float acc[MT][NT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  TileStager<BM, NWG> sta;
  TileStager<BN, NWG> stb;
  ScaleStager<BM, NWG> ssa;
  ScaleStager<BN, NWG> ssb;
  sta.init(lda, i0, I - 1, lw, lane);
  stb.init(ldb, j0, j0 + BN - 1, lw, lane);
  ssa.init(i0, I - 1, lw, lane);
  ssb.init(j0, j0 + BN - 1, lw, lane);
  auto stage_all = [&](int lbl, uint8_t* buf) {
    const int64_t lb = lb0 + lbl;
    sta.issue(A + i0 * lda + lb * BK, buf, lw);
    stb.issue(B + j0 * ldb + lb * BK, buf + BM * BK, lw);
    ssa.issue(SA + lb * ldsa + i0, reinterpret_cast<float*>(buf + C::kSaOff), lw, lane);
    if (SB_MODE == SB_ROWS) ssb.issue(SB + lb * ldsb + j0, ring + (lbl % C::kRing) * BN, lw, lane);
  };

  uint4 qa[2][MT], qb[2][NT];   // raw codes of two K slices (software pipeline)
  v8h fa[MT][2], fb[NT][2];     // converted operands of the slice being multiplied
  v16f p[MT][NT];               // block products
  auto load_slice = [&](const uint8_t* buf, int c, int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) qa[slot][mt] = lds16(buf, wm * WM + mt * 32 + rr, 4 * h + c);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qb[slot][nt] = lds16(buf + BM * BK, wn * WN + nt * 32 + rr, 4 * h + c);
    __builtin_amdgcn_sched_barrier(0x0006);
  };
  auto convert = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      fa[mt][0] = cvt8(qa[slot][mt].x, qa[slot][mt].y);
      fa[mt][1] = cvt8(qa[slot][mt].z, qa[slot][mt].w);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      fb[nt][0] = cvt8(qb[slot][nt].x, qb[slot][nt].y);
      fb[nt][1] = cvt8(qb[slot][nt].z, qb[slot][nt].w);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          p[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[nt][k], fa[mt][k], p[mt][nt], 0, 0, 0);
  };

  // Block lb of this group from `cur` (its slice 0 already in registers), as
  // in block_gemm_f16_kernel with double buffering: slices 1..3 read one ahead
  // of the multiply; after the block-end barrier `cur` is refilled with block
  // lb + 2 and slice 0 of block lb + 1 is read from `nxt` while the last slice
  // is multiplied.
  auto step = [&](uint8_t* cur, const uint8_t* nxt, int lb) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p[mt][nt] = v16f{};
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      load_slice(cur, c + 1, (c + 1) & 1);
      convert(c & 1);
      multiply();
    }
    convert(1);
    const float* lsa = reinterpret_cast<const float*>(cur + C::kSaOff);
    float sa[MT];                  // A scale of this lane's output row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa[mt] = lsa[wm * WM + mt * 32 + rr];
    const float sblk = (SB_MODE == SB_BLOCK) ? SB[(j0 / 128) * nLBtot + lb0 + lb] : 1.0f;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    if (lb + NS < nLB) stage_all(lb + NS, cur);
    if (lb + 1 < nLB) load_slice(nxt, 0, 0);
    multiply();
    float4 sbr[NT][4];             // SB_ROWS: B scales of output columns 8q + 4h + u
    const float* lsb = ring + (lb % C::kRing) * BN;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sbr[nt][q] = (SB_MODE == SB_ROWS) ? *reinterpret_cast<const float4*>(lsb + wn * WN + nt * 32 + 8 * q + 4 * h)
                                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float srow = (SB_MODE == SB_BLOCK) ? sa[mt] * sblk : sa[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float cs[4] = {sbr[nt][q].x, sbr[nt][q].y, sbr[nt][q].z, sbr[nt][q].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sc = (SB_MODE == SB_ROWS) ? srow * cs[u] : srow;
            acc[mt][nt][4 * q + u] = fmaf(p[mt][nt][4 * q + u], sc, acc[mt][nt][4 * q + u]);
          }
        }
    }
  };

  // Prologue: both stages of this group, wait for its first block.
  stage_all(0, lds0);
  if (nLB > 1) stage_all(1, lds1);
  if (nLB > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kVmemPerBlock));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  load_slice(lds0, 0, 0);
  for (int lb = 0; lb < nLB; lb += 2) {
    step(lds0, lds1, lb);
    if (lb + 1 < nLB) step(lds1, lds0, lb + 1);
  }

  // The second group's accumulators, lane-major (one 1 KB run per wave store),
  // through its own stage buffers: sub-tile row mt = 0 into the first, 1 into
  // the second.  Then the first group adds them (its own value first) and
  // stores the tile; the second group is done.
  lds_barrier();
  if (grp == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float* dst = reinterpret_cast<float*>(mt == 0 ? g1s0 : g1s1) + (lw * NT * 4) * 256 + lane * 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(dst + (nt * 4 + q) * 256) =
              make_float4(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
    }
  }
  lds_barrier();
  if (grp == 1) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float* src = reinterpret_cast<const float*>(mt == 0 ? g1s0 : g1s1) + (lw * NT * 4) * 256 + lane * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 o = *reinterpret_cast<const float4*>(src + (nt * 4 + q) * 256);
        acc[mt][nt][4 * q] += o.x;
        acc[mt][nt][4 * q + 1] += o.y;
        acc[mt][nt][4 * q + 2] += o.z;
        acc[mt][nt][4 * q + 3] += o.w;
      }
  }

  // Epilogue of the first group, one 32-row band at a time through its own
  // stage buffers (no other wave uses them any more).
  {
    using Bd = Band<OUT, WN>;
    uint8_t* region = band_region<32 * Bd::RS, C::kBufBytes, NS, NWG>(g0s0, g0s1, g0s1, lw);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* v = &acc[mt][nt][4 * q];
          uint8_t* pp = region + rr * Bd::RS + (nt * 32 + 8 * q + 4 * h) * Bd::ESZ;
          if (OUT == OUT_BF16) {
            *reinterpret_cast<uint2*>(pp) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
          } else {
            *reinterpret_cast<float4*>(pp) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      store_band<OUT, WN, 32>(region, lane, Cout, ldc, i0 + wm * WM + mt * 32, j0 + wn * WN, I);
    }
  }
}

// FP8 matrix-core path: one workgroup per output tile, the exact path's
// pipeline with the block product formed by v_mfma_f32_32x32x64_f8f6f4 on the
// E4M3 codes themselves (two per 32x32 sub-tile and block, no conversion).
template <int BM, int BN, int WM, int WN, int SB_MODE, int OUT, int NW, int NS, int S, bool PLANES>
__global__ __launch_bounds__(64 * NW, (NW == 4 && NS == 2) ? 2 : 1) void block_gemm_fp8_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ SB, int64_t ldsb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN,
    float* __restrict__ part, unsigned* __restrict__ cnt) {
  using C = Cfg<BM, BN, WM, WN, SB_MODE, PREC_FP8, NW, NS>;
  constexpr int MT = WM / 32, NT = WN / 32;
  // One distinct LDS object per pipeline stage (see the file comment).
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NS == 3 ? C::kBufBytes : 16];
  __shared__ __attribute__((aligned(16))) float sb_ring[SB_MODE == SB_ROWS ? C::kRing * BN : 4];
  __shared__ int split_flag;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int tm, tn, split;
  const int tile = map_tile<group_rows<BM>(), S>(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn, split);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int nLBtot = (int)(L / BK);
  const int lb0 = nLBtot * split / S;
  const int nLB = nLBtot * (split + 1) / S - lb0;   // this split's scale blocks
  // Lane l: row (l % 32) of a 32x32 sub-tile; half h = l / 32 holds K bytes
  // [64h, 64h + 64) of the block, and MFMA kh (0, 1) of the block takes the 32
  // bytes at 64h + 32kh (16-byte chunks 4h + 2kh and 4h + 2kh + 1).  A and B
  // use the same K order, so the sum is unchanged.  As in the exact path the
  // MFMA gets the B fragment first: lane l holds output row (l % 32) and, in
  // accumulator 4q + u, output column 8q + 4h + u.
  const int h = lane >> 5, rr = lane & 31;

  float acc[MT][NT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  TileStager<BM, NW> sta;
  TileStager<BN, NW> stb;
  ScaleStager<BM, NW> ssa;
  ScaleStager<BN, NW> ssb;
  sta.init(lda, i0, I - 1, wave, lane);
  stb.init(ldb, j0, j0 + BN - 1, wave, lane);
  ssa.init(i0, I - 1, wave, lane);
  ssb.init(j0, j0 + BN - 1, wave, lane);
  auto stage_all = [&](int lbl, uint8_t* buf) {
    const int64_t lb = lb0 + lbl;
    sta.issue(A + i0 * lda + lb * BK, buf, wave);
    stb.issue(B + j0 * ldb + lb * BK, buf + BM * BK, wave);
    ssa.issue(SA + lb * ldsa + i0, reinterpret_cast<float*>(buf + C::kSaOff), wave, lane);
    if (SB_MODE == SB_ROWS) ssb.issue(SB + lb * ldsb + j0, sb_ring + (lbl % C::kRing) * BN, wave, lane);
  };

  v8i fa[2][MT], fb[2][NT];   // codes of two K halves (software pipeline)
  v16f p[MT][NT];             // block products
  auto load_half = [&](const uint8_t* buf, int kh, int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * WM + mt * 32 + rr;
      const uint4 lo = lds16(buf, row, 4 * h + 2 * kh), hi = lds16(buf, row, 4 * h + 2 * kh + 1);
      fa[slot][mt] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = wn * WN + nt * 32 + rr;
      const uint4 lo = lds16(buf + BM * BK, row, 4 * h + 2 * kh), hi = lds16(buf + BM * BK, row, 4 * h + 2 * kh + 1);
      fb[slot][nt] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  auto multiply = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        // E4M3 x E4M3 (format selectors 0, 0), no block scaling in the MFMA.
        p[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[slot][nt], fa[slot][mt], p[mt][nt],
                                                                    0, 0, 0, 0, 0, 0);
  };

  // Block lb from `cur` (its first half already in registers): the second
  // half is read while the first is multiplied; then the wave waits for its
  // share of block lb + 1, the workgroup synchronises, `cur` is refilled with
  // block lb + NS and the first half of block lb + 1 is read from `nxt` -- all
  // while the second half is multiplied.  The block's scales are read into
  // registers before `cur` can be refilled.
  auto step = [&](uint8_t* cur, const uint8_t* nxt, int lb) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p[mt][nt] = v16f{};
    load_half(cur, 1, 1);
    multiply(0);
    const float* lsa = reinterpret_cast<const float*>(cur + C::kSaOff);
    float sa[MT];                  // A scale of this lane's output row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa[mt] = lsa[wm * WM + mt * 32 + rr];
    const float sblk = (SB_MODE == SB_BLOCK) ? SB[((j0 + wn * WN) / 128) * nLBtot + lb0 + lb] : 1.0f;
    if (NS == 3 && lb + 2 < nLB)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kVmemPerBlock));   // block lb+1 landed, lb+2 may fly
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    if (lb + NS < nLB) stage_all(lb + NS, cur);
    if (lb + 1 < nLB) load_half(nxt, 0, 0);
    multiply(1);
    float4 sbr[NT][4];             // SB_ROWS: B scales of output columns 8q + 4h + u
    const float* lsb = sb_ring + (lb % C::kRing) * BN;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sbr[nt][q] = (SB_MODE == SB_ROWS) ? *reinterpret_cast<const float4*>(lsb + wn * WN + nt * 32 + 8 * q + 4 * h)
                                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    // Rescale-accumulate: acc += P * SA(row) * SB.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float srow = (SB_MODE == SB_BLOCK) ? sa[mt] * sblk : sa[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float cs[4] = {sbr[nt][q].x, sbr[nt][q].y, sbr[nt][q].z, sbr[nt][q].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sc = (SB_MODE == SB_ROWS) ? srow * cs[u] : srow;
            acc[mt][nt][4 * q + u] = fmaf(p[mt][nt][4 * q + u], sc, acc[mt][nt][4 * q + u]);
          }
        }
    }
  };

  // Prologue: fill every buffer, wait for block 0, read its first half.
  const int pre = nLB < NS ? nLB : NS;
  stage_all(0, lds0);
  if (pre > 1) stage_all(1, lds1);
  if (NS == 3 && pre > 2) stage_all(2, lds2);
  if (NS == 3 && pre > 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::kVmemPerBlock));
  else if (pre > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kVmemPerBlock));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  load_half(lds0, 0, 0);
  if (NS == 2) {
    for (int lb = 0; lb < nLB; lb += 2) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds0, lb + 1);
    }
  } else {
    for (int lb = 0; lb < nLB; lb += 3) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds2, lb + 1);
      if (lb + 2 < nLB) step(lds2, lds0, lb + 2);
    }
  }

  if (S > 1 && !PLANES) {
    // Split-K, as in the exact path: partial tiles stored lane-major, the last
    // split to arrive adds them in split order.
    constexpr int kWave = MT * NT * 16 * 64;    // floats per wave and split
    float* mine = part + ((int64_t)(tile * S + split) * NW + wave) * kWave + lane * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(mine + ((mt * NT + nt) * 4 + q) * 256) =
              make_float4(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
    if (!split_arrive<S>(cnt + tile, t, &split_flag)) return;
    add_partials<S, MT, NT>(acc, part + ((int64_t)tile * S * NW + wave) * kWave + lane * 4, NW * kWave, split);
  }

  // Epilogue through LDS, one 32-row band at a time (as in the exact path).
  lds_barrier();
  {
    using Bd = Band<OUT, WN>;
    static_assert(!PLANES || (S > 1 && OUT == OUT_F32), "partial planes are FP32");
    // Small-grid split: this split's partial goes to plane `split` of the
    // workspace ([S][I][ldc] FP32); add_planes_kernel adds the planes.
    void* dst = PLANES ? static_cast<void*>(static_cast<float*>(Cout) + (int64_t)split * I * ldc) : Cout;
    uint8_t* region = band_region<32 * Bd::RS, C::kBufBytes, NS, NW>(lds0, lds1, lds2, wave);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* v = &acc[mt][nt][4 * q];
          uint8_t* pp = region + rr * Bd::RS + (nt * 32 + 8 * q + 4 * h) * Bd::ESZ;
          if (OUT == OUT_BF16) {
            *reinterpret_cast<uint2*>(pp) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
          } else {
            *reinterpret_cast<float4*>(pp) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      store_band<OUT, WN, 32>(region, lane, dst, ldc, i0 + wm * WM + mt * 32, j0 + wn * WN, I);
    }
  }
}

// Plain BF16 GEMM  C[i, j] = sum_l A[i, l] B[j, l]  (both operands BF16,
// contraction-contiguous), the comparator for the block-scaled FP8 GEMMs on
// the same shapes.  Same structure as the exact path: 64-element K stages of
// 128-byte rows staged straight into LDS (three buffers), K slices read one
// ahead of the multiply, v_mfma_f32_32x32x16_bf16 accumulating directly into
// the FP32 accumulators (no per-block scale), transposed sub-tiles and the same
// epilogue.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int BK16 = 64;   // BF16 elements per K stage (128 bytes per row)

template <int BM, int BN, int WM, int WN, int OUT, int NW, int NS>
__global__ __launch_bounds__(64 * NW, (NW == 4 && NS == 2) ? 2 : 1) void bf16_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN) {
  constexpr int WGN = BN / WN;
  constexpr int MT = WM / 32, NT = WN / 32;
  static_assert((BM / WM) * WGN == NW, "one wave per WM x WN sub-tile");
  constexpr int kBuf = (BM + BN) * BK;   // bytes per stage: 128-byte rows
  constexpr int kVmem = TileStager<BM, NW>::kLoads + TileStager<BN, NW>::kLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NS == 3 ? kBuf : 16];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int tm, tn, split;
  map_tile<group_rows<BM>(), 1>(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn, split);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = wave / WGN, wn = wave % WGN;
  const int nLB = (int)(L / BK16);
  // Lane l: row (l % 32) of a 32x32 sub-tile; half h = l / 32 holds elements
  // [32h, 32h + 32) of the stage; slice c (0..3) is the 8 elements at 32h + 8c,
  // one MFMA operand.  Output layout as in the exact FP8 path.
  const int h = lane >> 5, rr = lane & 31;

  v16f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v16f{};

  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(A);
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(B);
  TileStager<BM, NW> sta;
  TileStager<BN, NW> stb;
  sta.init(lda * 2, i0, I - 1, wave, lane);
  stb.init(ldb * 2, j0, j0 + BN - 1, wave, lane);
  auto stage_all = [&](int lb, uint8_t* buf) {
    sta.issue(Ab + i0 * lda * 2 + (int64_t)lb * BK, buf, wave);
    stb.issue(Bb + j0 * ldb * 2 + (int64_t)lb * BK, buf + BM * BK, wave);
  };
  uint4 qa[2][MT], qb[2][NT];
  auto load_slice = [&](const uint8_t* buf, int c, int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) qa[slot][mt] = lds16(buf, wm * WM + mt * 32 + rr, 4 * h + c);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qb[slot][nt] = lds16(buf + BM * BK, wn * WN + nt * 32 + rr, 4 * h + c);
  };
  auto multiply = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, qb[slot][nt]),
                                                               __builtin_bit_cast(v8bf, qa[slot][mt]), acc[mt][nt], 0, 0, 0);
  };
  auto step = [&](uint8_t* cur, const uint8_t* nxt, int lb) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      load_slice(cur, c + 1, (c + 1) & 1);
      multiply(c & 1);
    }
    if (NS == 3 && lb + 2 < nLB)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kVmem));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // The slice-3 registers must hold their data before `cur` is refilled.
    lds_barrier();
    if (lb + NS < nLB) stage_all(lb + NS, cur);
    // Slice 3 sits in slot 1; slice 0 of the next stage goes to slot 0.
    if (lb + 1 < nLB) load_slice(nxt, 0, 0);
    multiply(1);
  };
  const int pre = nLB < NS ? nLB : NS;
  stage_all(0, lds0);
  if (pre > 1) stage_all(1, lds1);
  if (NS == 3 && pre > 2) stage_all(2, lds2);
  if (NS == 3 && pre > 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kVmem));
  else if (pre > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kVmem));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  load_slice(lds0, 0, 0);
  if (NS == 2) {
    for (int lb = 0; lb < nLB; lb += 2) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds0, lb + 1);
    }
  } else {
    for (int lb = 0; lb < nLB; lb += 3) {
      step(lds0, lds1, lb);
      if (lb + 1 < nLB) step(lds1, lds2, lb + 1);
      if (lb + 2 < nLB) step(lds2, lds0, lb + 2);
    }
  }
  // Epilogue through LDS, one 32-row band at a time (as in the exact path).
  lds_barrier();
  {
    using Bd = Band<OUT, WN>;
    uint8_t* region = band_region<32 * Bd::RS, kBuf, NS, NW>(lds0, lds1, lds2, wave);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& v = acc[mt][nt];
          uint8_t* p = region + rr * Bd::RS + (nt * 32 + 8 * q + 4 * h) * Bd::ESZ;
          if (OUT == OUT_BF16) {
            *reinterpret_cast<uint2*>(p) = make_uint2(bf16x2(v[4 * q], v[4 * q + 1]), bf16x2(v[4 * q + 2], v[4 * q + 3]));
          } else {
            *reinterpret_cast<float4*>(p) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          }
        }
      store_band<OUT, WN, 32>(region, lane, Cout, ldc, i0 + wm * WM + mt * 32, j0 + wn * WN, I);
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(256) void fill_zero_kernel(void* __restrict__ C, int64_t rows, int64_t cols, int64_t ldc) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    if (OUT == OUT_BF16) static_cast<uint16_t*>(C)[r * ldc + c] = 0;
    else static_cast<float*>(C)[r * ldc + c] = 0.0f;
  }
}

__global__ __launch_bounds__(256) void clear_u32_kernel(unsigned* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Sum of the S partial planes of a small-grid split, in split order (plane 0
// + plane 1 + ... + plane S-1), then the output epilogue: FP32, BF16 (round
// to nearest even) or FP32 added to the values already in C.  part holds
// [S][I][J] FP32 (plane stride I * J); one thread handles 4 consecutive
// columns of a row, loading all S planes before adding.
template <int OUT, int S>
__global__ __launch_bounds__(256) void add_planes_kernel(const float* __restrict__ part, int64_t I, int64_t J,
                                                         void* __restrict__ C, int64_t ldc) {
  const int64_t per_row = J / 4, n = I * per_row, plane = I * J;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += (int64_t)gridDim.x * 256) {
    const int64_t i = v / per_row, j = (v - i * per_row) * 4;
    const float* p = part + i * J + j;
    float4 t[S];
#pragma unroll
    for (int sp = 0; sp < S; ++sp) t[sp] = *reinterpret_cast<const float4*>(p + sp * plane);
    float4 sum = t[0];
#pragma unroll
    for (int sp = 1; sp < S; ++sp) {
      sum.x += t[sp].x; sum.y += t[sp].y; sum.z += t[sp].z; sum.w += t[sp].w;
    }
    if (OUT == OUT_BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + i * ldc + j) =
          make_uint2(bf16x2(sum.x, sum.y), bf16x2(sum.z, sum.w));
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(C) + i * ldc + j);
      if (OUT == OUT_F32_ACC) {
        const float4 old = *dst;
        sum.x += old.x; sum.y += old.y; sum.z += old.z; sum.w += old.w;
      }
      *dst = sum;
    }
  }
}

constexpr int kCUs = 256;   // MI355X compute units

template <int BM, int BN, int WM, int WN, int SB_MODE, int OUT, int PREC, int NW, int NS, int S, bool PLANES = false>
void launch_cfg(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, float* part, unsigned* cnt, hipStream_t st) {
  const int tilesM = (int)((I + BM - 1) / BM), tilesN = (int)(J / BN);
  const int nUnits = tilesM * tilesN * S;
  if (PREC == PREC_F16) {
    hipLaunchKernelGGL((block_gemm_f16_kernel<BM, BN, WM, WN, SB_MODE, OUT, NW, NS, S, PLANES>), dim3(nUnits), dim3(64 * NW),
                       0, st, A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN, part, cnt);
  } else {
    hipLaunchKernelGGL((block_gemm_fp8_kernel<BM, BN, WM, WN, SB_MODE, OUT, NW, NS, S, PLANES>), dim3(nUnits), dim3(64 * NW),
                       0, st, A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN, part, cnt);
  }
}

// Small-grid split: S kernels' worth of partial planes from one launch of
// 128 x 128 tiles x S splits, then add_planes_kernel.
template <int SB_MODE, int OUT, int PREC, int S>
void launch_planes_s(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                     const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                     int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, float* part, hipStream_t st) {
  launch_cfg<128, 128, 64, 64, SB_MODE, OUT_F32, PREC, 4, 2, S, true>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L,
                                                                      part, J, nullptr, nullptr, st);
  const int64_t n = I * (J / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL((add_planes_kernel<OUT, S>), dim3(blocks), dim3(256), 0, st, part, I, J, C, ldc);
}

template <int SB_MODE, int OUT, int PREC>
void launch_planes(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                   const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                   int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, const SplitPlan& plan, hipStream_t st) {
  if (plan.splits == 2)
    launch_planes_s<SB_MODE, OUT, PREC, 2>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan.part, st);
  else if (plan.splits == 4)
    launch_planes_s<SB_MODE, OUT, PREC, 4>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan.part, st);
  else
    launch_planes_s<SB_MODE, OUT, PREC, 8>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan.part, st);
}

// Tile choice: a split plan runs the split on 256 x 128 tiles (split in two,
// FP8BLK_GEMM_SPLIT2) or on 128 x 128 tiles into partial planes (split 2, 4 or
// 8 ways, the default for small grids); otherwise 256 x 128 output tiles (8 waves of 64 x 64,
// triple-buffered LDS, one workgroup per CU) when they fill every CU for a
// whole number of rounds, else 128 x 128 tiles: on the exact path with at
// most one tile per CU, 8 waves in two K groups (block_gemm_f16_kgroups_kernel),
// otherwise 4 waves, double-buffered, two workgroups per CU, whose finer
// granularity keeps every CU busy in a partial last round.
template <int SB_MODE, int OUT, int PREC>
void launch_prec(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                 const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                 int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, const SplitPlan& plan, hipStream_t st) {
  if (plan.splits > 1 && plan.split_big_tiles)
    launch_cfg<256, 128, 64, 64, SB_MODE, OUT, PREC, 8, 3, 2>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc,
                                                              plan.part, plan.counters, st);
  else if (plan.splits > 1)
    launch_planes<SB_MODE, OUT, PREC>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan, st);
  else if (plan.big_tiles)
    launch_cfg<256, 128, 64, 64, SB_MODE, OUT, PREC, 8, 3, 1>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc,
                                                              nullptr, nullptr, st);
  else if (PREC == PREC_F16 && plan.kgroups) {
    const int tilesM = (int)((I + 127) / 128), tilesN = (int)(J / 128);
    hipLaunchKernelGGL((block_gemm_f16_kgroups_kernel<SB_MODE, OUT>), dim3(tilesM * tilesN), dim3(512), 0, st,
                       A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN);
  }
  else
    launch_cfg<128, 128, 64, 64, SB_MODE, OUT, PREC, 4, 2, 1>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc,
                                                              nullptr, nullptr, st);
}

template <int OUT>
void launch_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t I, int64_t J, int64_t L,
                 void* C, int64_t ldc, hipStream_t st) {
  if (((I + 255) / 256) * (J / 128) >= kCUs) {
    const int tm = (int)((I + 255) / 256), tn = (int)(J / 128);
    hipLaunchKernelGGL((bf16_gemm_kernel<256, 128, 64, 64, OUT, 8, 3>), dim3(tm * tn), dim3(512), 0, st,
                       A, lda, B, ldb, I, L, C, ldc, tm, tn);
  } else {
    const int tm = (int)((I + 127) / 128), tn = (int)(J / 128);
    hipLaunchKernelGGL((bf16_gemm_kernel<128, 128, 64, 64, OUT, 4, 2>), dim3(tm * tn), dim3(256), 0, st,
                       A, lda, B, ldb, I, L, C, ldc, tm, tn);
  }
}

}  // namespace

// Workspace layout of the split in two (FP8BLK_GEMM_SPLIT2): a fixed 64 KiB
// region of 4-byte arrival counters (one per output tile, so at most
// kMaxSplitTiles tiles are split), then two FP32 partial tiles of 256 x 128
// per output tile.  The counter region does not depend on the shape, so one
// workspace can serve problems of different shapes in turn: no problem's
// partial tiles ever overlap another problem's counters, and every call leaves
// the counters it used at zero.  The small-grid split needs no counters; it
// leaves the counter region untouched and puts S FP32 partial planes of the
// I x J output after it, so a workspace whose counters are zero stays valid for
// either plan in any order.
constexpr int64_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxSplitTiles = kCounterBytes / 4;

size_t split_workspace_bytes(int64_t I, int64_t J, int splits) {
  if (splits <= 1) return 0;
  const int64_t tiles = ((I + 255) / 256) * (J / 128);
  if (tiles > kMaxSplitTiles) return 0;
  return (size_t)kCounterBytes + (size_t)tiles * splits * 256 * 128 * 4;
}

// The split a problem uses by default, given room for it in the workspace.
// Grids of at most kCUs / 4 output tiles of 128 x 128 (e.g. a 256-token
// forward GEMM into 2048 features: 32 tiles, each contracting 16 scale blocks
// on a CU of its own while 224 CUs idle) are split along the contraction into
// S = 8, 4 or 2: the largest S with S * tiles <= kCUs and at least two scale
// blocks per split.  The splits write FP32 partial planes and a second kernel
// adds them in split order (an in-kernel last-arriver sum was slower here:
// each workgroup's agent-scope release writes back its XCD's L2, and the last
// split read the other seven partial tiles on its own).  Larger grids are not
// split: splitting the contraction in
// two was measured on the layer's under-filled shapes -- the o and down weight
// gradients, 128 and 384 tiles of 256 x 128 -- and was slower than the
// unsplit kernels there (59 against 50 us and 160 against 128 us at 4096
// tokens): each split pays the tile prologue and epilogue, the partial tiles'
// round trip and one L2 write-back, more than the fuller CUs gain.  The split
// in two on 256 x 128 tiles stays available on request (FP8BLK_GEMM_SPLIT2).
int small_grid_splits(int64_t I, int64_t J, int64_t L) {
  const int64_t tiles = ((I + 127) / 128) * (J / 128);
  const int64_t nLB = L / 128;
  if (tiles > kCUs / 4) return 1;
  int s = 8;
  while (s > 1 && (tiles * s > kCUs || nLB < 2 * s)) s /= 2;
  return s;
}

size_t small_split_workspace_bytes(int64_t I, int64_t J, int splits) {
  if (splits <= 1) return 0;
  return (size_t)kCounterBytes + (size_t)splits * (size_t)I * (size_t)J * 4;
}

SplitPlan plan_split(int64_t I, int64_t J, int64_t L, void* ws, size_t ws_bytes, bool force) {
  SplitPlan p;
  const int64_t big = ((I + 255) / 256) * (J / 128);
  p.big_tiles = big >= kCUs && big % kCUs == 0;
  // At most one 128 x 128 tile per CU (a 2048 x 2048 weight gradient: 256
  // tiles): two K groups of 4 waves per tile, so that every SIMD runs two
  // waves (measured on the O weight gradient over 4096 tokens: 48 -> 43 us).
  // Grids with more tiles already run two 4-wave workgroups per CU, where
  // 8-wave tiles were slower (the down projection's: 114 -> 123 us).
  const int64_t tiles128 = ((I + 127) / 128) * (J / 128);
  p.kgroups = !p.big_tiles && tiles128 <= kCUs && (L / 128) % 2 == 0;
  if (force) {
    const size_t need = split_workspace_bytes(I, J, 2);
    if (L / 128 >= 2 && need > 0 && ws != nullptr && ws_bytes >= need) {
      p.splits = 2;
      p.split_big_tiles = true;
    }
  } else {
    const int s = small_grid_splits(I, J, L);
    const size_t need = small_split_workspace_bytes(I, J, s);
    if (s > 1 && need > 0 && ws != nullptr && ws_bytes >= need) p.splits = s;
  }
  if (p.splits > 1) {
    p.kgroups = false;
    p.counters = p.split_big_tiles ? static_cast<unsigned*>(ws) : nullptr;
    p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes);
  }
  return p;
}

void launch_block_gemm(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                       const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb, int sb_mode,
                       int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int out_mode,
                       int prec, const SplitPlan& plan, hipStream_t st) {
  if (L == 0) {   // empty contraction: the product is zero
    if (out_mode == OUT_F32_ACC) return;
    const int64_t n = I * J;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (out_mode == OUT_BF16)
      hipLaunchKernelGGL(fill_zero_kernel<OUT_BF16>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    else
      hipLaunchKernelGGL(fill_zero_kernel<OUT_F32>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    return;
  }
#define FP8BLK_GEMM_CASE(SBM, OM)                                                              \
  if (sb_mode == SBM && out_mode == OM) {                                                      \
    if (prec == PREC_FP8)                                                                            \
      launch_prec<SBM, OM, PREC_FP8>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan, st); \
    else                                                                                             \
      launch_prec<SBM, OM, PREC_F16>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, plan, st); \
    return;                                                                                    \
  }
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_F32)
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_BF16)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32_ACC)
#undef FP8BLK_GEMM_CASE
}

void launch_clear_u32(unsigned* p, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(clear_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n);
}

void launch_bf16_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int out_mode, hipStream_t st) {
  if (L == 0) {
    const int64_t n = I * J;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (out_mode == OUT_BF16)
      hipLaunchKernelGGL(fill_zero_kernel<OUT_BF16>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    else
      hipLaunchKernelGGL(fill_zero_kernel<OUT_F32>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    return;
  }
  if (out_mode == OUT_BF16)
    launch_bf16<OUT_BF16>(A, lda, B, ldb, I, J, L, C, ldc, st);
  else
    launch_bf16<OUT_F32>(A, lda, B, ldb, I, J, L, C, ldc, st);
}

}  // namespace fp8blk
