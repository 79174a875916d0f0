// MFMA kernels of the quintic Newton-Schulz iteration (gfx950, bf16 in, fp32
// accumulate): parameter-golf walkthrough Part 1 (A = X X^T, B = b A + c A A,
// X = a X + B X) with the coefficients of the "Muon Custom Sizing"
// walkthrough, section 2.3, which also names a symmetric kernel for X X^T.
//
// Products C[i][j] = sum_k P[i][k] Q[k][j] over an oriented padded iterate
// X [mp][np]:
//   Gram   A  = scale X X^T            P = X rows, Q = X^T: both read as
//                                      k-contiguous rows of X            (K = np)
//   poly   B' = a I + b A + c A A      P = Q = A                         (K = mp)
//   bx     X' = scale B' X             P = B', Q = X                     (K = mp)
// The a X term of the update is carried by the diagonal of B'
// (a X + B X = (a I + B) X), so the B X epilogue reads nothing.
//
// A and B' are symmetric (their kernel computes only the upper-triangle tiles
// ti <= tj and writes each off-diagonal tile a second time, transposed, so
// the stored matrices are exactly symmetric).  Hence their row panels equal
// their column panels, and poly and bx read every operand as a k-major panel
// (k rows of 2 BT contiguous bytes: whole cache lines), like X in B X.
//
// ACCURATE precision keeps B' and X as bf16 hi + lo pairs; its B X product
// Bh Xh + Bh Xl + Bl Xh is one product over a reduction three times as long,
// [Bh | Bh | Bl] [Xh; Xl; Xh], whose segments are read from the three pairs
// of planes in turn (so every tiling accumulates a 32 x 32 output block in
// the same order, and a stage holds two operand tiles, as for FAST).
//
// Tiling: a workgroup computes a BT x BT output tile, BT = 256 with 8 waves of
// 128 x 64 (two per SIMD) or BT = 128 with 4 waves of 64 x 64, each wave's
// part a grid of v_mfma_f32_32x32x16_bf16 accumulators.  K steps by 32
// through a ring of four LDS stages (256-wide tiles and every B X tile; the
// 128-wide Gram and polynomial tiles use two stages of 64, below), operand
// slices fetched straight into LDS with buffer_load_dwordx4 ... lds (no
// staging registers).  Once per step, just before its last 16-deep
// sub-slice, every wave waits for its own loads of the next slice and then at
// a barrier; the loads of slice k + 3 go into the stage just freed, spread
// over that sub-slice one instruction per two MFMAs.  Fragments of sub-slice
// u + 1 are read from LDS while the MFMAs of u run.  A k-contiguous operand
// tile sits in LDS as rows x 32 bf16, 16-byte chunk index XOR-swizzled by the
// row; a k-major tile as it lies in memory (BK k-rows x BT columns, 16-byte
// chunks XOR-swizzled by 4 (row % 4)), its fragments read with
// ds_read_b64_tr_b16, two per fragment, which transposes on the way.  Both
// layouts are conflict-free for their reads; the swizzle is applied on the
// global side of the DMA.
//
// Epilogue: 32 rows of a wave's accumulators at a time are staged in LDS as
// fp32 and read back row by row, so global stores write 128-byte row segments
// (a wave tile's 64 columns).  The mirror tile of a symmetric output is staged as bf16 and
// read back with ds_read_b64_tr_b16, two reads handing each lane 8
// consecutive rows of one column for a 16-byte store.
//
// MFMA 32x32x16 lane layout: lane l supplies row (l % 32) of its operand and
// 8 consecutive k values starting at 8 (l / 32); result element (r, c) of a
// 32 x 32 block sits in lane 32 ((r / 4) % 2) + c, register 4 (r / 8) + r % 4.
// The kernels pass the column operand first, so each lane holds 4 consecutive
// output columns of one output row.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8 bytes addressed by lanes 4 e + i / 4, for e = 0..3.  With
// lane L addressing row rb + L / 4, columns cb + 4 (L % 4) .. + 3 of a
// row-major tile, lane i gets rows rb .. rb + 3 of column cb + i.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <set>
#include <tuple>
#include <type_traits>
#include <vector>

#include "muon_internal.hpp"
#include "ns_schedule.hpp"

namespace muon {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// LDS of gfx950 has 64 banks of 4 bytes: a 16-byte read by 16 lanes, or an
// 8-byte read by 32 lanes, is conflict-free when the lanes cover 256
// distinct-bank bytes.
//
// A k-contiguous operand tile in LDS: rows of BK bf16 (2 BK bytes, BK / 8
// chunks of 16 bytes); chunk c of row r is stored at chunk c ^ f(r) with
// f(r) = (r / RP) mod (BK / 8), RP = 256 / (2 BK) rows per 256 bytes.  Any 16
// consecutive rows then cover all 64 banks for 16-byte fragment reads.
template <int BK>
__device__ __forceinline__ int swz(int row) {
    return (row / (128 / BK)) & (BK / 8 - 1);
}
template <int BK>
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * (2 * BK) + ((chunk ^ swz<BK>(row)) << 4);
}

// Pipeline (K slice BK, NS LDS stages):
//  * ring: BK = 32 in NS = 4 stages; the wait and barrier of a step come
//    before its last sub-slice, and slice k + 3 is fetched into the stage
//    just freed (it lands two steps later).  256-wide tiles, and the B X
//    product at any width.
//  * two stages: BK = 64 in NS = 2; slice k + 1 is fetched during step k and
//    waited for at the end of the step.  128-wide Gram and polynomial tiles
//    (two workgroups per CU): the 128-byte k-contiguous rows of X X^T are
//    whole cache lines (a 64-byte row costs the same L1 miss as a full
//    line), and the other workgroup on the CU covers the first fragment
//    reads of each step.
//
// Waves: a 64-wide tile is computed by 4 waves of 32 x 32, a 128-wide tile by
// 4 waves of 64 x 64, a 256-wide tile by 8 waves of 128 x 64 (two per SIMD,
// 128 accumulator registers each).  The 64-wide tiles are for batches too
// small to fill the CUs, whose time is the chain of dependent products: a
// shorter tile shortens every link.
// With one wave per SIMD, the DMA issue, the vmcnt wait and the barrier of
// each step leave the matrix core idle for about a quarter of the loop; a
// second wave on the SIMD issues its MFMAs in those gaps.
template <int BT, bool RING>
struct TileCfg {
    static constexpr int NW = BT == 256 ? 8 : 4;    // waves
    static constexpr int TWR = BT / 2;              // wave tile rows
    static constexpr int TWC = 2 * BT / NW;         // wave tile columns
    static constexpr int FA = TWR / 32;             // 32x32 blocks per wave: rows
    static constexpr int FB = TWC / 32;             //                        columns
    static constexpr int WC = BT / TWC;             // waves across the tile's columns
    static constexpr int BK = RING ? 32 : 64;       // K slice per stage
    static constexpr int NS = RING ? 4 : 2;         // LDS stages
    static constexpr int OP_BYTES = BT * BK * 2;    // one operand tile
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor of `bytes` bytes at `base` (stride 0; loads past the
// end return zero without accessing memory, so `bytes` = 0 makes a load that
// fetches nothing but still counts in vmcnt).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{static_cast<int>(static_cast<uint32_t>(b)), static_cast<int>((b >> 32) & 0xffffu),
                 static_cast<int>(bytes), 0x00020000};
}

// One buffer_load_dwordx4 ... lds: lane L's 16 bytes at rsrc + voff + soff go to
// LDS byte address lds + 16 L.  It is issued as inline assembly so that the
// compiler does not track it: the compiler would otherwise make every
// transposing LDS read (which carries no alias information) wait for all of
// this wave's outstanding DMA, which collapses the pipeline.  The kernel
// orders DMA and LDS reads itself with explicit vmcnt waits and barriers.
//
// Inline assembly is also outside the compiler's hazard recognizer.  A
// vector memory instruction that reads an SGPR shortly after a VALU wrote it
// (v_readfirstlane, or v_readlane restoring a spilled SGPR) can use the
// SGPR's previous value and fetch from the wrong place: measured on gfx950
// with in-bounds buffer loads, 40-77% of loads directly after the
// v_readfirstlane of their offset and 2-52% one instruction later (varying
// from run to run) used the old offset; none from two instructions between
// on.  VALU_SGPR (the caller's descriptor or
// offset comes from v_readfirstlane) puts five wait states, the figure
// documented for gfx9, before the load.  The build scans the generated code
// and rejects any other DMA within five wait states of a VALU write of its
// SGPRs.  A scalar write of M0 right before the load needs none.
template <bool VALU_SGPR = false>
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, char* lds) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));
    if constexpr (VALU_SGPR)
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(m0), "v"(voff), "s"(rsrc),
                     "s"(soff) : "memory");
    else
        asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(m0), "v"(voff), "s"(rsrc), "s"(soff)
                     : "memory");
}

// An R x BK slice of a k-contiguous matrix fetched straight into LDS by the
// NW waves of the workgroup: one instruction of one wave fills 1 KB (lane L
// writes bytes [16 L, 16 L + 16)), i.e. 512 / BK rows of BK / 8 chunks.  The
// lane whose LDS slot is (row, physical chunk p) fetches logical chunk
// p ^ swz(row).
template <int R, int BK_, int NW>
struct RowDma {
    static constexpr int BK = BK_;
    static constexpr int CPR = BK / 8;               // chunks per row
    static constexpr int RPW = 64 / CPR;             // rows per 1 KB window
    static constexpr int PW = R / RPW / NW;          // windows per wave
    static_assert(PW >= 1 && PW * RPW * NW == R, "slice splits evenly over the waves");
    const void* base;                   // the matrix; its buffer descriptor is built in load()
    uint32_t bytes;
    uint32_t voff[PW];

    __device__ __forceinline__ void init(const void* base_, uint32_t bytes_, int64_t ld, int row0, int tid) {
        base = base_;
        bytes = bytes_;
        const int w = tid >> 6, l = tid & 63;
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            const int row = RPW * (w * PW + q) + l / CPR;
            const int chunk = (l % CPR) ^ swz<BK>(row);
            voff[q] = static_cast<uint32_t>(((int64_t)(row0 + row) * ld + chunk * 8) * 2);
        }
    }
    // Window q of this wave (1 KB) of the slice at K offset k0 (k0 < 0: an
    // empty range, which fetches nothing).
    __device__ __forceinline__ void load_q(char* lds, int k0, int q, int tid) const {
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool live = k0 >= 0;
        dma16(make_rsrc(base, live ? bytes : 0u), voff[q], static_cast<uint32_t>((live ? k0 : 0) * 2),
              lds + (w * PW + q) * 1024);
    }
};

// A BK x C slice (BK k-rows, C columns) of a column-contiguous matrix in its
// own layout: rows of 2C bytes, 16-byte chunk c of row r stored at chunk
// c ^ (4 (r % 4)), so the 4 rows x 64 bytes that 32 lanes of a transposing
// read touch land in 4 distinct 64-byte bank groups.
// One DMA instruction of one wave fills 1 KB = 512 / C rows.
template <int C>
__device__ __forceinline__ int col_swz(int row) {
    // C >= 128: 16 or more chunks per row, XOR 4 (row % 4); C = 64 (8 chunks):
    // XOR 4 ((row / 2) % 2), so rows r and r + 2, which share banks, differ
    return C >= 128 ? (row & 3) << 2 : ((row >> 1) & 1) << 2;
}
template <int C>
__device__ __forceinline__ int col_off(int row, int col) {
    return row * (2 * C) + (((col >> 3) ^ col_swz<C>(row)) << 4) + (((col >> 2) & 1) << 3);
}

template <int C, int BK_, int NW, int LO_SEG = -1>
struct ColDma {
    static constexpr int BK = BK_;
    static constexpr int ROWS_PER_WIN = 512 / C;
    static constexpr int PW = BK / ROWS_PER_WIN / NW;  // 1 KB windows per wave
    static_assert(PW >= 1 && PW * ROWS_PER_WIN * NW == BK, "slice splits evenly over the waves");
    // LO_SEG >= 0: the reduction runs over three segments of seg_k rows each,
    // segment LO_SEG read from `lo` and the other two from `base` (same
    // layout); k0 counts over all of them.
    const void* base;
    const void* lo;
    uint32_t bytes;
    uint32_t ldb;                                      // row pitch in bytes
    int seg_k;
    uint32_t voff[PW];

    __device__ __forceinline__ void init(const void* base_, uint32_t bytes_, int64_t ld, int col0, int tid,
                                         const void* lo_ = nullptr, int seg_k_ = 0) {
        base = base_;
        lo = lo_;
        bytes = bytes_;
        ldb = static_cast<uint32_t>(ld * 2);
        seg_k = seg_k_;
        const int w = tid >> 6, l = tid & 63;
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            const int row = ROWS_PER_WIN * (w * PW + q) + l / (C / 8);
            const int chunk = (l % (C / 8)) ^ col_swz<C>(row);
            voff[q] = static_cast<uint32_t>(((int64_t)row * ld + col0 + chunk * 8) * 2);
        }
    }
    // As RowDma::load_q (k0 < 0: an empty range).
    __device__ __forceinline__ void load_q(char* lds, int k0, int q, int tid) const {
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool live = k0 >= 0;
        if (!live) k0 = 0;
        if constexpr (LO_SEG >= 0) {
            // k0 is uniform: the segment and its base are kept in scalar registers
            const int s = (k0 >= seg_k) + (k0 >= 2 * seg_k);
            const uint64_t bp = reinterpret_cast<uint64_t>(s == LO_SEG ? lo : base);
            // readfirstlane returns int: widen through uint32_t (a sign extension
            // would set the high address word whenever bit 31 is set)
            const uint32_t b_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bp)));
            const uint32_t b_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bp >> 32)));
            const uint64_t bs = uint64_t(b_lo) | (uint64_t(b_hi) << 32);
            const uint32_t soff = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(k0 - s * seg_k) * ldb);
            dma16<true>(make_rsrc(reinterpret_cast<const void*>(bs), live ? bytes : 0u), voff[q], soff,
                        lds + (w * PW + q) * 1024);
        } else {
            dma16(make_rsrc(base, live ? bytes : 0u), voff[q], static_cast<uint32_t>(k0) * ldb, lds + (w * PW + q) * 1024);
        }
    }
};

// The operands of one kernel: NA tiles for the output rows and NB tiles for
// the output columns, each either k-contiguous rows (RowDma) or k-major
// columns (ColDma).
template <int BT, int NA, int NB, typename ALoader, typename BLoader, bool SHARE_B = false>
struct Operands {
    ALoader a[NA];
    BLoader b[NB];
    // SHARE_B (symmetric products): with b_empty set, the column operand's
    // loads fetch nothing (it is read from the row operand's tile).
    bool b_empty = false;
    static constexpr int OP_BYTES = BT * ALoader::BK * 2;   // one operand tile
    static constexpr int STAGE = (NA + NB) * OP_BYTES;
    static constexpr int WINDOWS = NA * ALoader::PW + NB * BLoader::PW;   // DMA instructions per wave
    __device__ __forceinline__ static char* a_tile(char* stage, int i) { return stage + i * OP_BYTES; }
    __device__ __forceinline__ static char* b_tile(char* stage, int j) {
        return stage + (NA + j) * OP_BYTES;
    }
    // DMA instruction w (0 <= w < WINDOWS) of this wave for the slice at k0
    // (k0 < 0: an empty range).
    __device__ __forceinline__ void load_window(char* stage, int k0, int w, int tid) const {
        constexpr int PA = ALoader::PW, PB = BLoader::PW;
        if (w < NA * PA) {
            a[w / PA].load_q(a_tile(stage, w / PA), k0, w % PA, tid);
        } else {
            const int v = w - NA * PA;
            b[v / PB].load_q(b_tile(stage, v / PB), SHARE_B && b_empty ? -1 : k0, v % PB, tid);
        }
    }
    __device__ __forceinline__ void load(char* stage, int k0, int tid) const {
#pragma unroll
        for (int w = 0; w < WINDOWS; ++w) load_window(stage, k0, w, tid);
    }
};

// One fragment (a 32-wide block at base, one 16-deep sub-slice ks) of an
// operand.  From k-contiguous rows: one 16-byte read.  From a k-major tile:
// two transposing reads (k rows ks*16 + 8 (l / 32) + 0..3 and + 4..7 of
// index l % 32 of the block).
template <bool KMAJOR, int BT, int BK>
__device__ __forceinline__ bf16x8 load_frag(const char* S, int base, int ks, int tid) {
    const int lane = tid & 63;
    if constexpr (!KMAJOR) {
        return *reinterpret_cast<const bf16x8*>(
            S + lds_off<BK>(base + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
        const int L = lane & 15, grp = (lane >> 4) & 1;
        const int row = 16 * ks + 8 * (lane >> 5) + (L >> 2);
        const int col = base + grp * 16 + 4 * (L & 3);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(S + col_off<BT>(row, col)));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(S + col_off<BT>(row + 4, col)));
        const i16x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
}

// The fragments of one sub-slice, read in the order the MFMAs consume them
// (a0 with b0 .. b(FB-1), then a1, a2, ...), so the reads issued last have the
// most MFMAs of the next sub-slice to complete behind.  With DMA, the W loads
// of a stage (into `next`, K offset k1) are issued in between: fragment g of
// the G fragment reads that carry them (this call's first fragment is number
// g0) issues the windows w with w G in [g W, (g + 1) W).  The reads are placed
// one per MFMA, so the DMA instructions are spread over the MFMA stream
// instead of stalling the wave in a burst when the address queue fills.
template <int FA, int FB, bool KMAJOR_A, bool KMAJOR_B, int BT, int BK, bool DMA = false, int G = 1,
          typename Ops = void>
__device__ __forceinline__ void load_frags(const char* As, const char* Bs, int wr0, int wc0, int ks,
                                           bf16x8 (&a)[FA], bf16x8 (&b)[FB], int tid, const Ops* ops = nullptr,
                                           char* next = nullptr, int k1 = 0, int g0 = 0) {
    auto dma_after = [&](int fi) {
        if constexpr (DMA) {
            constexpr int W = Ops::WINDOWS;
            const int g = g0 + fi;
#pragma unroll
            for (int w = 0; w < W; ++w)
                if (w * G >= g * W && w * G < (g + 1) * W) ops->load_window(next, k1, w, tid);
        }
    };
    a[0] = load_frag<KMAJOR_A, BT, BK>(As, wr0, ks, tid);
    dma_after(0);
#pragma unroll
    for (int j = 0; j < FB; ++j) {
        b[j] = load_frag<KMAJOR_B, BT, BK>(Bs, wc0 + j * 32, ks, tid);
        dma_after(1 + j);
    }
#pragma unroll
    for (int i = 1; i < FA; ++i) {
        a[i] = load_frag<KMAJOR_A, BT, BK>(As, wr0 + i * 32, ks, tid);
        dma_after(FB + i);
    }
}

template <int FA, int FB>
__device__ __forceinline__ void mfma_block(const bf16x8 (&a)[FA], const bf16x8 (&b)[FB], f32x16 (&acc)[FA][FB]) {
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
}

// Interleaves the NM MFMAs of one sub-slice with the NREAD LDS reads issued
// beside them (the fragments of the next sub-slice).  Square 4-wave tiles
// alternate read and MFMA groups; the 8-wave tiles spread their reads evenly
// ahead of each MFMA (12 reads over 8 MFMAs for k-major operands).
template <int NM, int NREAD, int M>
__device__ __forceinline__ void spread_reads() {
    constexpr int nr = ((M + 1) * NREAD) / NM - (M * NREAD) / NM;
    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);    // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // one MFMA
    if constexpr (M + 1 < NM) spread_reads<NM, NREAD, M + 1>();
}
template <int NM, int NREAD, bool SPREAD>
__device__ __forceinline__ void interleave() {
    if constexpr (!SPREAD) {
#pragma unroll
        for (int t = 0; t < NREAD; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, NM / NREAD, 0);     // MFMA
        }
    } else {
        spread_reads<NM, NREAD, 0>();
    }
}

// Waits until at most N of this wave's DMA instructions are outstanding, then
// for every wave of the workgroup.  A bare s_barrier does not drain the
// outstanding loads the way __syncthreads does; the empty asm statements keep
// the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_dma_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(imm);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int FA, int FB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FA][FB]) {
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int s = 0; s < 16; ++s) acc[i][j][s] = 0.f;
}

__device__ __forceinline__ u32x2 pack4(const uint16_t (&h)[4]) {
    u32x2 w;
    w[0] = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
    w[1] = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
    return w;
}

// Workgroups of one launch are handed to the 8 XCDs round-robin (w -> XCD
// w % 8).  Renumbering them so that each XCD gets one contiguous range of
// logical tiles keeps the operand panels of a matrix in a single XCD's L2.
__device__ __forceinline__ uint32_t xcd_logical(uint32_t w, uint32_t total) {
    const uint32_t q = total >> 3, r = total & 7, x = w & 7;
    return x * q + (x < r ? x : r) + (w >> 3);
}

// Epilogue staging, per wave and per 32-row chunk of its wave tile (TW
// columns).
// fp32 chunk: rows of TW floats, 16-byte chunk index XOR (row % 16), so the
// MFMA-layout writes (16 rows, one chunk) and the row-contiguous reads (one
// row, 16 chunks) are both conflict-free.
template <int TW>
__device__ __forceinline__ int f32_off(int row, int col) {
    return row * (TW * 4) + (((col >> 2) ^ (row & (TW >= 64 ? 15 : TW / 4 - 1))) << 4);
}
// bf16 chunk for the mirror store: rows of TW bf16, 16-byte chunk index XOR
// an even row function chosen so that the transposing reads (rows 0-3 and
// 8-11 of a 16-row group, two adjacent chunks) hit distinct banks.
template <int TW>
__device__ __forceinline__ int mir_off(int row, int col) {
    const int f = TW == 128 ? 2 * ((row & 3) | (((row >> 3) & 1) << 2))
                : TW == 64  ? 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1))
                            : 2 * ((row >> 1) & 1);
    return row * (TW * 2) + (((col >> 3) ^ f) << 4) + (((col >> 2) & 1) << 3);
}

// bf16 chunk of the B X epilogue: rows of TW bf16 (CH = TW / 8 chunks of 16
// bytes), chunk index XOR (row % CH) and the two 8-byte halves of a chunk
// swapped on rows CH..2 CH - 1.  The MFMA-layout writes (8 bytes by each of
// 32 rows x 2 lanes) then cover 64 distinct banks for TW = 128, and the
// row reads (16 bytes, CH lanes per row) each cover a whole row.
template <int TW>
__device__ __forceinline__ int bst_off(int row, int col) {
    constexpr int CH = TW / 8;
    return row * (TW * 2) + (((col >> 3) ^ (row & (CH - 1))) << 4) + ((((col >> 2) & 1) ^ ((row / CH) & 1)) << 3);
}

enum Kind { kGram = 0, kPoly = 1, kPolySplit = 2, kBx = 3, kBxSplit = 4 };

// One product of a launch: a batch of same-shaped blocks.  A launch may carry
// up to kMaxProblems of them (same kind, same tiling), enumerated one after
// the other, so that several parameter shapes fill the CUs together.
constexpr int kMaxProblems = 4;

struct GemmProblem {
    const uint16_t* p[2];     // row operands (hi, lo): X, A or B'
    const uint16_t* q[2];     // column operands (hi, lo): X or A or X
    uint16_t* out[2];         // row-major output (hi, lo)
    // The first iteration's Frobenius norm, from the trace of X X^T: the
    // Gram writes one partial per 32-row block of each block's diagonal
    // (trace + blk * trace_stride), the polynomial and B X read them.  Null
    // in later iterations.
    float* trace;
    int64_t trace_stride;
    int ntrace;               // partials per block: padded rows / 32
    int64_t p_stride, q_stride, out_stride;
    int64_t K;                // reduction length (row pitch of k-contiguous operands)
    int64_t ldq;              // row pitch of a k-major column operand
    int64_t ldo;              // output row pitch
    uint32_t p_bytes, q_bytes;
    // Tile enumeration (of 256-wide tiles in quadrant mode): block-major;
    // within a block the upper triangle row by row (symmetric) or ti fastest.
    int T;                    // symmetric: tiles per side
    uint32_t tiles_i;         // full: row tiles per block
    uint32_t tiles;           // tiles per block
    uint32_t first;           // index of this problem's first tile in the launch
};

struct GemmArgs {
    GemmProblem pr[kMaxProblems];
    int n;                    // problems in this launch
    uint32_t total;           // workgroups of this launch
    uint32_t* status;         // null, or the call's two status words, which workgroup 0 clears
    // Quadrant mode (128-wide kernel finishing the last partial round of a
    // 256-wide tiling): workgroup L computes quadrant L % 4 of 256-wide tile
    // big_base + L / 4.
    uint32_t quad, big_base;
    float ca, cb, cc, eps;
};

// One output tile of one product, its pointers already offset to the block.
struct TileJob {
    const uint16_t* p[2];     // row operands (hi, lo): X, A or B'
    const uint16_t* q[2];     // column operands (hi, lo): X, A or X
    uint16_t* out[2];         // row-major output (hi, lo)
    // The first iteration's norm partials of this block (one per 32 rows of
    // the diagonal: the Gram writes them, the polynomial and B X read them),
    // or null in later iterations.
    float* trace;
    int ntrace;
    uint32_t p_bytes, q_bytes;
    int64_t K;                // reduction length (row pitch of k-contiguous operands)
    int64_t ldq;              // row pitch of a k-major column operand
    int64_t ldo;              // output row pitch
    int ti, tj;               // tile row and column (in tiles of BT)
};

// LDS bytes of one tile of KIND at width BT (the operand stages; the
// epilogue staging reuses them).
template <int BT, int KIND>
constexpr bool ring_pipeline() {
    return BT != 128 || KIND == kBx || KIND == kBxSplit;
}
template <int KIND, int BT>
constexpr int tile_lds_bytes() {
    using Cfg = TileCfg<BT, ring_pipeline<BT, KIND>()>;
    return Cfg::NS * 2 * Cfg::OP_BYTES;
}

struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// 1 / (sqrt(sum of the n partials) + eps), the same value in every lane and
// every caller: lane k adds partials k, k + 64, ... in order, then the lanes'
// sums are added in a fixed tree to lane 0 and broadcast.
__device__ __forceinline__ float norm_inverse(const float* part, int n, float eps) {
    const int lane = static_cast<int>(threadIdx.x & 63);
    float v = 0.f;
    for (int i = lane; i < n; i += 64) v += part[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_down(v, off, 64);
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
    return 1.0f / (sqrtf(tot) + eps);
}

// Sum of the diagonal of a 32 x 32 accumulator block, valid in lane 0, in a
// fixed order.  Lane l holds row l % 32 and, in element 4 g + e, column
// 8 g + 4 (l / 32) + e, so diagonal entry c sits in lane c + 32 ((c / 4) % 2),
// element 4 (c / 8) + c % 4.
__device__ __forceinline__ float diag_sum32(const f32x16& acc, int lane) {
    const int c = lane & 31;
    const bool has = ((c >> 2) & 1) == (lane >> 5);
    const int idx = ((c >> 3) << 2) | (c & 3);
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
        if (q == idx) v = acc[q];
    v = has ? v : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_down(v, off, 64);
    return v;
}

// The operand loaders of one tile of KIND at width BT.
template <int KIND, int BT>
struct TileTypes {
    using Cfg = TileCfg<BT, ring_pipeline<BT, KIND>()>;
    static constexpr bool SPLIT_IN = KIND == kBxSplit;                // hi/lo planes of both operands
    // Operand layouts: X X^T reads rows of X (k-contiguous).  A and B' are
    // symmetric, so their row panels are also column panels, and X of B X is
    // k-major as stored.  A k-major slice row is a whole 2 BT-byte run of full
    // cache lines, where a k-contiguous slice row is only 2 BK bytes; a
    // k-contiguous fragment is one 16-byte LDS read per lane, a k-major one
    // two transposing reads.  Measured per launch: the 128-wide polynomial
    // runs about 6% faster k-contiguous (two-stage pipeline, BK = 64), the
    // 64-wide one 20% slower, the 256-wide one within noise in the loop; B X
    // with k-contiguous B' rows is up to 13% slower.
    static constexpr bool KMAJOR_A = KIND != kGram && !((KIND == kPoly || KIND == kPolySplit) && BT == 128);
    static constexpr bool KMAJOR_B = KMAJOR_A;
    static constexpr int BK = Cfg::BK, NW = Cfg::NW;
    // split B X: the row operand reads its lo plane in segment 2, the column operand in segment 1
    using ALoader = typename std::conditional<KMAJOR_A, ColDma<BT, BK, NW, SPLIT_IN ? 2 : -1>, RowDma<BT, BK, NW>>::type;
    using BLoader = typename std::conditional<KMAJOR_B, ColDma<BT, BK, NW, SPLIT_IN ? 1 : -1>, RowDma<BT, BK, NW>>::type;
    using Ops = Operands<BT, 1, 1, ALoader, BLoader, KIND == kGram || KIND == kPoly || KIND == kPolySplit>;
    static constexpr int STAGE = Ops::STAGE;

    __device__ __forceinline__ static void init(Ops& ops, const TileJob& a, int tid) {
        const int row0 = a.ti * BT, col0 = a.tj * BT;
        if constexpr (SPLIT_IN) {
            // segments: Bh Xh, Bh Xl, Bl Xh
            ops.a[0].init(a.p[0], a.p_bytes, a.K, row0, tid, a.p[1], static_cast<int>(a.K));
            ops.b[0].init(a.q[0], a.q_bytes, a.ldq, col0, tid, a.q[1], static_cast<int>(a.K));
        } else {
            ops.a[0].init(a.p[0], a.p_bytes, a.K, row0, tid);   // K = ld (square when k-major)
            ops.b[0].init(a.q[0], a.q_bytes, KMAJOR_B ? a.ldq : a.K, col0, tid);
        }
    }
};

// Computes one BT x BT output tile with the NW waves of the workgroup,
// using `lds` (tile_lds_bytes<KIND, BT>() bytes) for the operand stages and
// the epilogue.  All LDS traffic of the previous use of `lds` must be
// finished (a barrier) before the call.  Each wave calls hook() once in its
// epilogue, after the last global load it waits for (so that a memory
// operation the hook issues is not waited for by the rest of the tile).
template <int KIND, int BT, bool OPAQUE_TID = false, typename Hook = NoHook, bool SHARE_DIAG = true>
__device__ __forceinline__ void gemm_tile(const TileJob& a, char* lds, float ca, float cb, float cc, float eps,
                                          const Hook& hook = Hook()) {
    // In a loop over tiles the thread index is made opaque per tile, so that
    // the compiler does not hoist the lane-dependent address arithmetic of
    // every product out of the loop (and spill it).
    int tid = static_cast<int>(threadIdx.x);
    if constexpr (OPAQUE_TID) asm volatile("" : "+v"(tid));
    using TT = TileTypes<KIND, BT>;
    using Cfg = typename TT::Cfg;
    constexpr int FB = Cfg::FB, TWR = Cfg::TWR, TWC = Cfg::TWC, NW = Cfg::NW;
    constexpr bool SYM = KIND == kGram || KIND == kPoly || KIND == kPolySplit;
    constexpr bool POLY = KIND == kPoly || KIND == kPolySplit;
    constexpr bool SPLIT_IN = TT::SPLIT_IN;
    constexpr bool SPLIT_OUT = KIND == kPolySplit || KIND == kBxSplit;
    constexpr bool KMAJOR_A = TT::KMAJOR_A, KMAJOR_B = TT::KMAJOR_B;
    constexpr int NSEG = SPLIT_IN ? 3 : 1;            // reduction segments (split B X: Bh Xh, Bh Xl, Bl Xh)
    constexpr int BK = Cfg::BK;
    using Ops = typename TT::Ops;
    constexpr int STAGE = Ops::STAGE;
    constexpr int LDS_BYTES = Cfg::NS * STAGE;
    static_assert(LDS_BYTES == tile_lds_bytes<KIND, BT>(), "LDS size");
    const int ti = a.ti, tj = a.tj;
    const int row0 = ti * BT, col0 = tj * BT;
    const int wave = tid >> 6;

    Ops ops;
    TT::init(ops, a, tid);
    // A diagonal tile of a symmetric product reads the same rows as both
    // operands (X X^T: rows of X; A A: rows of A): only the row operand is
    // fetched, the column operand's loads go through an empty range (same
    // instruction count, so the same waits), and the column fragments are
    // read from the row operand's tile.  SHARE_DIAG = false keeps both
    // fetches: the ACCURATE persistent loop, whose split B'X phase ran
    // 2-7% slower on 2048- and 4096-row blocks when the diagonal tiles
    // before it were shortened (measured; the per-product launches and the
    // FAST loop gain).
    const bool same_ops = SYM && SHARE_DIAG && ti == tj;
    if constexpr (SYM) ops.b_empty = same_ops;
    const int bsel = same_ops ? 0 : Ops::OP_BYTES;

    // The first iteration scales by s^-1 = 1 / (|X|_F + eps) (B X) or uses
    // s^-2, s^-4 (the polynomial of the unscaled X X^T).  The norm partials
    // are loaded with the operand prologue, so that the epilogue waits for
    // no global load of its own.
    float sc = 1.0f;
    if constexpr (KIND != kGram) {
        if (a.trace != nullptr) sc = norm_inverse(a.trace, a.ntrace, eps);
    }
    if constexpr (POLY) {
        const float s2 = sc * sc;
        cb *= s2;
        cc *= s2 * s2;
    }

    // The K loop and epilogue of one wave, which computes FA x FB blocks of
    // 32 x 32 at rows wr0, columns wc0 of the tile, and stores their mirror
    // (the transposed block at the transposed place) for its first
    // `mirror_chunks` 32-row chunks.  Every
    // wave runs the same K loop structure (one wait, barrier and stage of DMA
    // per step) whatever its FA.
    const auto body = [&](auto fa_tag, const int wr0, const int wc0, const int mirror_chunks) {
    constexpr int FA = decltype(fa_tag)::value;
    f32x16 acc[FA][FB];
    zero_acc<FA, FB>(acc);

    // A K step is U sub-slices (16 deep); the fragments of sub-slice u + 1 are
    // read from LDS while the MFMAs of u run.
    constexpr int NS = Cfg::NS;
    constexpr int KS = BK / 16;
    constexpr int U = KS;
    static_assert(U % 2 == 0, "fragment ping-pong restarts at 0 each step");
    constexpr int NREAD = (KMAJOR_A ? 2 * FA : FA) + (KMAJOR_B ? 2 * FB : FB);
    constexpr int NM = FA * FB;
    constexpr bool SPREAD = NW == 8 || NM < NREAD;
    constexpr int W = Ops::WINDOWS;
    const int nk = static_cast<int>(NSEG * a.K / BK);
    bf16x8 fa[2][FA], fb[2][FB];
    auto frags = [&](const char* st, int u, bf16x8 (&xa)[FA], bf16x8 (&xb)[FB]) {
        load_frags<FA, FB, KMAJOR_A, KMAJOR_B, BT, BK>(Ops::a_tile(const_cast<char*>(st), 0),
                                              const_cast<char*>(st) + bsel, wr0, wc0, u, xa, xb, tid);
    };

    if constexpr (NS >= 3) {
        // Ring: slice kt lives in stage kt % NS.  Just before the last
        // sub-slice of step kt every wave waits for its own loads of slice
        // kt + 1 and then at a barrier, after which stage (kt - 1) % NS is
        // free (step kt - 1 consumed all its reads) and slice kt + NS - 1 is
        // fetched into it, spread over the last sub-slice, whose reads are
        // the first fragments of slice kt + 1.  Every step issues exactly one
        // stage of loads, so the wait count is fixed: past the last slice the
        // loads name K offset -1, which the loaders turn into an empty
        // buffer range (no memory access; the stage, never read, gets zeros).
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) ops.load(lds + st * STAGE, st < nk ? st * BK : -1, tid);
        wait_dma_and_barrier<(NS - 2) * W>();
        frags(lds, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            char* cur = lds + (kt % NS) * STAGE;
            char* nxt = lds + ((kt + 1) % NS) * STAGE;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = u & 1;
                if (u + 1 < U) {
                    frags(cur, u + 1, fa[c ^ 1], fb[c ^ 1]);
                } else {
                    // The sub-slice that waits, passes the barrier and issues
                    // the next stage's DMA runs at raised wave priority, so
                    // the SIMD's other wave does not delay the loads
                    // (measured 0.7% faster; raising it around the MFMAs
                    // instead was 3.7% slower).
                    __builtin_amdgcn_s_setprio(1);
                    wait_dma_and_barrier<(NS - 3) * W>();
                    const int kn = kt + NS - 1;
                    load_frags<FA, FB, KMAJOR_A, KMAJOR_B, BT, BK, true, FA + FB>(
                        Ops::a_tile(nxt, 0), nxt + bsel, wr0, wc0, 0, fa[c ^ 1], fb[c ^ 1], tid, &ops,
                        lds + (kn % NS) * STAGE, kn < nk ? kn * BK : -1, 0);
                }
                mfma_block<FA, FB>(fa[c], fb[c], acc);
                interleave<NM, NREAD, SPREAD>();
                __builtin_amdgcn_sched_barrier(0);
                if (u + 1 == U) __builtin_amdgcn_s_setprio(0);
            }
        }
    } else {
        // Two stages: slice kt + 1 is fetched into the other stage during step
        // kt, spread over its first U - 1 sub-slices, and waited for at the
        // end of the step, where a barrier also frees stage kt % 2.
        ops.load(lds, 0, tid);
        wait_dma_and_barrier<0>();
        for (int kt = 0; kt < nk; ++kt) {
            char* cur = lds + (kt & 1) * STAGE;
            char* nxt = lds + ((kt + 1) & 1) * STAGE;
            const int k1 = kt + 1 < nk ? (kt + 1) * BK : -1;
            frags(cur, 0, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = u & 1;
                if (u + 1 < U) {
                    load_frags<FA, FB, KMAJOR_A, KMAJOR_B, BT, BK, true, (U - 1) * (FA + FB)>(
                        Ops::a_tile(cur, 0), cur + bsel, wr0, wc0, u + 1,
                        fa[c ^ 1], fb[c ^ 1], tid, &ops, nxt, k1, u * (FA + FB));
                }
                mfma_block<FA, FB>(fa[c], fb[c], acc);
                if (u + 1 < U) interleave<NM, NREAD, SPREAD>();
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_dma_and_barrier<0>();
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): no DMA may land on the epilogue staging
    __syncthreads();

    // ---- epilogue, one 32-row chunk of the wave tile at a time: the fp32
    // accumulators go through LDS so that global stores (and the A reads of
    // the polynomial) cover whole row segments instead of the MFMA layout's
    // 4-column pieces of 32 rows.  All staging is wave-private; LDS accesses
    // of one wave complete in order, so no barrier is needed.
    const int lane = tid & 63;
    const int lr = lane & 31, lk = lane >> 5;
    if constexpr (KIND == kGram) {
        // The first iteration's norm partials: the traces of the 32 x 32
        // blocks on the block's diagonal, taken from the fp32 accumulators
        // (each such block lies in one wave's tile).
        if (a.trace != nullptr && ti == tj) {
#pragma unroll
            for (int i = 0; i < FA; ++i)
#pragma unroll
                for (int j = 0; j < FB; ++j)
                    if (wr0 + 32 * i == wc0 + 32 * j) {
                        const float v = diag_sum32(acc[i][j], lane);
                        if (lane == 0) a.trace[(row0 + wr0 + 32 * i) >> 5] = v;
                    }
        }
    }
    const uint16_t* amat = POLY ? a.p[0] : nullptr;
    uint16_t* out0 = a.out[0];
    uint16_t* out1 = SPLIT_OUT ? a.out[1] : nullptr;
    // Staging per wave: the fp32 chunk, and for a symmetric tile the bf16
    // chunk of the mirror store.  Without split outputs the bf16 chunk
    // overlays the fp32 one: bf16 row r occupies the bytes of fp32 row r / 2,
    // which every lane has read (in an earlier or the same read-back
    // instruction, and one wave's LDS accesses complete in order) before any
    // lane writes there.  The split products keep both bf16 planes apart.
    constexpr int ST_F32 = 32 * TWC * 4;
    constexpr int ST_BF = SYM ? 32 * TWC * 2 : 0;
    constexpr int WAVE_LDS = SPLIT_OUT ? ST_F32 + 2 * ST_BF : ST_F32;
    static_assert(NW * WAVE_LDS <= LDS_BYTES, "epilogue staging must fit in LDS");
    char* sf = lds + wave * WAVE_LDS;
    char* sb = SPLIT_OUT ? sf + ST_F32 : sf;
    char* sb_lo = sb + ST_BF;
    constexpr int LPR = TWC / 4;      // lanes per row on read-back (4 values each)
    constexpr int RPI = 64 / LPR;     // rows per read-back instruction
    const int rrow = lane / LPR, rcol = (lane % LPR) * 4;
    const int64_t gcol = col0 + wc0 + rcol;
    // The polynomial's A values of chunk i + 1 are loaded while chunk i is
    // finished (double buffer), so their latency is exposed once, not per row.
    constexpr int NT = 32 / RPI;      // read-back instructions per chunk
    u32x2 abuf[2][NT];
    auto load_a = [&](int i, u32x2 (&dst)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            dst[t] = *reinterpret_cast<const u32x2*>(amat + (int64_t)(row0 + wr0 + i * 32 + t * RPI + rrow) * a.ldo +
                                                     gcol);
    };
    if constexpr (POLY)
        load_a(0, abuf[0]);
    else
        hook();
#pragma unroll
    for (int i = 0; i < FA; ++i) {
        if constexpr (KIND == kBx) {
            // B X: the rounded bf16 values go through LDS (half the bytes of
            // fp32 staging) and leave as 16-byte pieces of rows.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < FB; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint16_t hb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) hb[e] = f32_to_bf16(acc[i][j][g * 4 + e] * sc);
                    *reinterpret_cast<u32x2*>(sf + bst_off<TWC>(lr, j * 32 + g * 8 + lk * 4)) = pack4(hb);
                }
            __builtin_amdgcn_sched_barrier(0);
            constexpr int CH = TWC / 8, RPB = 64 / CH;
            const int brow = lane / CH, bch = lane % CH;
#pragma unroll
            for (int t = 0; t < 32 / RPB; ++t) {
                const int rr = t * RPB + brow;
                u32x4 v = *reinterpret_cast<const u32x4*>(sf + rr * (TWC * 2) + ((bch ^ (rr & (CH - 1))) << 4));
                if ((rr / CH) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
                *reinterpret_cast<u32x4*>(out0 + (int64_t)(row0 + wr0 + i * 32 + rr) * a.ldo + col0 + wc0 + 8 * bch) = v;
            }
            continue;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                 acc[i][j][g * 4 + 3]};
                *reinterpret_cast<f32x4*>(sf + f32_off<TWC>(lr, j * 32 + g * 8 + lk * 4)) = v;
            }
        if constexpr (POLY) {
            if (i + 1 < FA) load_a(i + 1, abuf[(i + 1) & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int rr = t * RPI + rrow;
            const int64_t grow = row0 + wr0 + i * 32 + rr;
            const int64_t o = grow * a.ldo + gcol;
            const f32x4 x = *reinterpret_cast<const f32x4*>(sf + f32_off<TWC>(rr, rcol));
            float am[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (POLY) {
                const u32x2 av = abuf[i & 1][t];
                am[0] = bf16_to_f32(uint16_t(av[0] & 0xffffu));
                am[1] = bf16_to_f32(uint16_t(av[0] >> 16));
                am[2] = bf16_to_f32(uint16_t(av[1] & 0xffffu));
                am[3] = bf16_to_f32(uint16_t(av[1] >> 16));
            }
            uint16_t hb[4], lb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v;
                if constexpr (POLY) {
                    v = fmaf(cc, x[e], cb * am[e]);
                    if (grow == gcol + e) v += ca;
                } else {
                    v = x[e] * sc;
                }
                hb[e] = f32_to_bf16(v);
                if constexpr (SPLIT_OUT) lb[e] = f32_to_bf16(v - bf16_to_f32(hb[e]));
            }
            *reinterpret_cast<u32x2*>(out0 + o) = pack4(hb);
            if constexpr (SPLIT_OUT) *reinterpret_cast<u32x2*>(out1 + o) = pack4(lb);
            if constexpr (SYM) {
                if (i < mirror_chunks) {
                    *reinterpret_cast<u32x2*>(sb + mir_off<TWC>(rr, rcol)) = pack4(hb);
                    if constexpr (SPLIT_OUT) *reinterpret_cast<u32x2*>(sb_lo + mir_off<TWC>(rr, rcol)) = pack4(lb);
                }
            }
        }
        // The polynomial's last wait for A values is above.
        if constexpr (POLY) {
            if (i + 1 == FA) hook();
        }
        if constexpr (SYM) {
            // Mirror: output row (col0 + wc0 + c) gets this chunk's 32 values of
            // column c.  Two transposing reads give lane L of 16-lane group g4
            // rows 8 g4 .. 8 g4 + 7 of column cb + L, stored as 16 bytes.
            if (i < mirror_chunks) {
                const int L = lane & 15, g4 = lane >> 4;
                const int srow = 8 * g4 + (L >> 2);
#pragma unroll
                for (int cb = 0; cb < TWC; cb += 16) {
                    const int scol = cb + 4 * (L & 3);
                    const int64_t o = (int64_t)(col0 + wc0 + cb + L) * a.ldo + row0 + wr0 + i * 32 + 8 * g4;
                    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(sb + mir_off<TWC>(srow, scol)));
                    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(sb + mir_off<TWC>(srow + 4, scol)));
                    *reinterpret_cast<i16x8*>(out0 + o) = i16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    if constexpr (SPLIT_OUT) {
                        const i16x4 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(sb_lo + mir_off<TWC>(srow, scol)));
                        const i16x4 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(sb_lo + mir_off<TWC>(srow + 4, scol)));
                        *reinterpret_cast<i16x8*>(out1 + o) =
                            i16x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
                    }
                }
            }
        }
    }
    };
    // A diagonal 256-wide tile of a symmetric product: its lower-left
    // quadrant is the transpose of the upper-right one, so no wave computes
    // it.  Waves 0-3 take the upper-right quadrant as 64 x 64 pieces and store
    // each piece twice (itself and, transposed, the lower-left quadrant).
    // Each diagonal 128 x 128 quadrant is symmetric too: the odd wave of its
    // pair (5, 7) takes its right 128 x 64 half and stores the upper 64 x 64
    // of it twice (itself and, transposed, the quadrant's lower-left block),
    // the even wave (4, 6) only its upper-left 64 x 64 diagonal block.  Wave
    // w shares a SIMD with wave w + 4, so the SIMDs issue 8, 12, 8 and 12 of
    // the 16 MFMA blocks per sub-slice (10 of 16 64 x 64 blocks executed in
    // all).  The mirrored blocks are bitwise the directly computed ones (the
    // same products, summed in the same order), and with fewer MFMAs the
    // tile draws less power: the 32 x 768x3072 NS call runs about 1% faster
    // than with the diagonal quadrants computed whole.
    if constexpr (SYM && NW == 8) {
        if (ti == tj) {
            const int q0 = (wave & 2) ? 128 : 0;
            if (wave < 4)
                body(std::integral_constant<int, 2>(), (wave >> 1) * 64, 128 + (wave & 1) * 64, 2);
            else if ((wave & 1) == 0)
                body(std::integral_constant<int, 2>(), q0, q0, 0);
            else
                body(std::integral_constant<int, 4>(), q0, q0 + 64, 2);
            return;
        }
    }
    body(std::integral_constant<int, Cfg::FA>(), (wave / Cfg::WC) * TWR, (wave % Cfg::WC) * TWC,
         SYM && ti != tj ? Cfg::FA : 0);
}

// Threads of a tile's workgroup.
template <int BT>
constexpr int tile_threads() {
    return 64 * TileCfg<BT, true>::NW;
}

template <int KIND, int BT>
__global__ __launch_bounds__(tile_threads<BT>()) void k_gemm(GemmArgs args) {
    constexpr bool SYM = KIND == kGram || KIND == kPoly || KIND == kPolySplit;
    constexpr bool SPLIT_IN = KIND == kBxSplit;
    constexpr bool SPLIT_OUT = KIND == kPolySplit || KIND == kBxSplit;
    __shared__ __attribute__((aligned(16))) char lds[tile_lds_bytes<KIND, BT>()];

    const uint32_t L = xcd_logical(blockIdx.x, args.total);
    const uint32_t tile_all = args.quad ? args.big_base + L / 4 : L;
    int pi = 0;
    for (int i = 1; i < args.n; ++i)
        if (tile_all >= args.pr[i].first) pi = i;
    const GemmProblem& a = args.pr[pi];
    const uint32_t tile = tile_all - a.first;
    const int64_t blk = tile / a.tiles;
    int ti, tj;
    {
        int id = static_cast<int>(tile % a.tiles);
        if constexpr (SYM) {
            int t = 0, len = a.T;
            while (id >= len) { id -= len; ++t; --len; }
            ti = t;
            tj = t + id;
        } else {
            ti = id % static_cast<int>(a.tiles_i);
            tj = id / static_cast<int>(a.tiles_i);
        }
        if (args.quad) {
            ti = 2 * ti + static_cast<int>((L >> 1) & 1);
            tj = 2 * tj + static_cast<int>(L & 1);
            if (SYM && ti > tj) return;   // lower quadrant of a diagonal tile: its mirror covers it
        }
    }
    TileJob j;
    j.p[0] = a.p[0] + blk * a.p_stride;
    j.p[1] = SPLIT_IN ? a.p[1] + blk * a.p_stride : nullptr;
    j.q[0] = a.q[0] + blk * a.q_stride;
    j.q[1] = SPLIT_IN ? a.q[1] + blk * a.q_stride : nullptr;
    j.out[0] = a.out[0] + blk * a.out_stride;
    j.out[1] = SPLIT_OUT ? a.out[1] + blk * a.out_stride : nullptr;
    j.trace = a.trace ? a.trace + blk * a.trace_stride : nullptr;
    j.ntrace = a.ntrace;
    j.p_bytes = a.p_bytes;
    j.q_bytes = a.q_bytes;
    j.K = a.K;
    j.ldq = a.ldq;
    j.ldo = a.ldo;
    j.ti = ti;
    j.tj = tj;
    if (args.status != nullptr && blockIdx.x == 0 && threadIdx.x < 2) args.status[threadIdx.x] = 0u;
    gemm_tile<KIND, BT>(j, lds, args.ca, args.cb, args.cc, args.eps);
}

// ---------------------------------------------------------------- persistent NS loop
// One launch runs every iteration of the Gram, polynomial and B X products of
// up to kMaxNsLoopProblems block batches, as 256-wide tiles.  Each workgroup
// (one per CU) takes the next item of its queue (an atomic head): a run of up
// to 16 consecutive tiles of one product of one block.  It waits until the
// block has completed every tile of the products before that one (done[block]
// reaches the item's count), computes the tiles and adds their number to
// done[block].  Items are listed in an order in which each depends only on
// items listed before it in the same queue, and an item is taken only by a
// running workgroup, so the lowest unfinished item can always proceed.
//
// Failure is loud.  A wait longer than spin_ticks sets the error word, and a
// workgroup that finds it set while waiting takes no further item.  The last
// workgroup to leave checks every block's counter: the final iterate of each
// block that did not complete all of its tiles is overwritten with NaN, and
// the number of such blocks and the error flags are added to the call's
// status words (which the caller can read back), so no result of an
// interrupted run passes for a valid one.
struct PersistProblem {
    const uint16_t* x0;       // iteration 0's input (oriented, padded)
    uint16_t* xb[2];          // ping-pong iterates: iteration t > 0 reads xb[t % 2] and
    uint16_t* xlast;          // writes xb[(t + 1) % 2]; the last iteration writes xlast
    uint16_t* xlo[2];         // ACCURATE: lo planes of the iterates (iteration t reads xlo[t % 2])
    uint16_t* a;
    uint16_t* b;
    uint16_t* blo;            // ACCURATE: lo plane of B'
    float* trace;             // iteration 0's norm partials (Gram writes, polynomial and B X read)
    int64_t trace_stride;     // floats between blocks' partials (a multiple of 32: 128-byte lines)
    uint32_t* done;           // [nb] completion counters, kSyncStride words apart
    int32_t mp, np;
    uint32_t first_blk;       // global index of its first block
    uint32_t nb;              // blocks
    uint32_t nsym, nbx;       // tiles per block: symmetric products, B X
};

struct PersistArgs {
    PersistProblem pr[kMaxNsLoopProblems];
    int n;
    int nq;                   // queues: 1, or 8 (a workgroup serves the queue of the XCD it runs on)
    int steps;                // iterations
    int inject;               // diagnostics: every workgroup sets the error word at its start
    const uint2* items;       // x = global block | (tiles - 1) << 28, y = first tile | product << 22 | iteration << 24
    uint32_t qbase[9];        // queue q is items[qbase[q], qbase[q + 1])
    uint32_t* sync;           // queue heads 0..7, then the error word and the exit counter
    uint32_t* status;         // the call's status words: [0] blocks left incomplete, [1] error flags
    uint64_t spin_ticks;      // longest dependency wait (ticks of the 100 MHz real-time counter)
    float ca, cb, cc, eps;
};

// Counters of the loop each sit on their own 128-byte line (kSyncStride
// words apart): queue heads 0..7, then the error word (word 0 of line 8) and
// the exit counter (word 1 of line 8), then one line per block.
constexpr uint32_t kSyncStride = 32;
constexpr uint32_t kSyncLines = 9;
constexpr uint32_t kItemEnd = 0xffffffffu;
constexpr uint32_t kBlockMask = 0x0fffffffu;   // item.x: block; the top 4 bits: tiles in the item - 1
// Items of the workgroup's queue held in LDS (a window from the queue index
// win0; wave 0 reloads it when an index passes its end).
constexpr uint32_t kLdsItems = 2048;

__device__ __forceinline__ uint32_t hw_xcc_id() {
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 15u;   // HW_REG_XCC_ID
}

// Run by the last workgroup to leave, with all its threads, once every other
// workgroup has left (so nothing else writes the iterates any more): each
// block whose counter shows fewer than all of its tiles gets NaN in its final
// iterate; the count and the error word go to the call's status words.
__device__ void ns_loop_verify(const PersistArgs& args, uint32_t* err, char* lds) {
    uint32_t* const s_bad = reinterpret_cast<uint32_t*>(lds);          // incomplete blocks of one round
    uint32_t* const s_cnt = reinterpret_cast<uint32_t*>(lds) + 512;    // their count
    const uint32_t tid = threadIdx.x;
    const PersistProblem& lastp = args.pr[args.n - 1];
    const uint32_t total = lastp.first_blk + lastp.nb;
    // Every other workgroup's completion counts were released by its exit
    // increment, which this workgroup's exit increment acquired.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t bad = 0;
    for (uint32_t base = 0; base < total; base += 512) {
        if (tid == 0) *s_cnt = 0;
        __syncthreads();
        const uint32_t g = base + tid;
        if (g < total) {
            int pi = 0;
            for (int i = 1; i < args.n; ++i)
                if (g >= args.pr[i].first_blk) pi = i;
            const PersistProblem& pr = args.pr[pi];
            const uint32_t expect = uint32_t(args.steps) * (2 * pr.nsym + pr.nbx);
            const uint32_t d =
                __hip_atomic_load(pr.done + kSyncStride * (g - pr.first_blk), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d != expect) s_bad[atomicAdd(s_cnt, 1u)] = g;
        }
        __syncthreads();
        const uint32_t nbad = *s_cnt;
        for (uint32_t k = 0; k < nbad; ++k) {
            const uint32_t g2 = s_bad[k];
            int pi = 0;
            for (int i = 1; i < args.n; ++i)
                if (g2 >= args.pr[i].first_blk) pi = i;
            const PersistProblem& pr = args.pr[pi];
            const int64_t elems = int64_t(pr.mp) * pr.np;
            u32x4* dst = reinterpret_cast<u32x4*>(pr.xlast + int64_t(g2 - pr.first_blk) * elems);
            const u32x4 nan4 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};   // bf16 quiet NaN
            for (int64_t e = tid; e < elems / 8; e += blockDim.x) dst[e] = nan4;
        }
        bad += nbad;
        __syncthreads();
    }
    if (tid == 0) {
        const uint32_t e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bad) __hip_atomic_fetch_add(args.status, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bad || e)
            __hip_atomic_fetch_or(args.status + 1, e | (bad ? 2u : 0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// SPLIT: ACCURATE precision (B' and X as hi + lo planes).
template <bool SPLIT>
__global__ __launch_bounds__(tile_threads<256>()) void k_ns_loop(PersistArgs args) {
    constexpr int LDS = tile_lds_bytes<kBx, 256>();
    static_assert(tile_lds_bytes<kGram, 256>() <= LDS && tile_lds_bytes<kPoly, 256>() <= LDS &&
                  tile_lds_bytes<kPolySplit, 256>() <= LDS && tile_lds_bytes<kBxSplit, 256>() <= LDS, "LDS size");
    static_assert(LDS + 8 * kLdsItems + 8 <= 160 * 1024, "LDS of a gfx950 workgroup");
    static_assert(LDS >= 513 * 4, "verification list fits in the tile LDS");
    __shared__ __attribute__((aligned(16))) char lds[LDS];
    __shared__ uint2 s_items[kLdsItems];
    __shared__ uint2 s_item;
    // The loop's control flow is uniform across the workgroup: wave 0 does the
    // queue and counter work, lane 0 alone issuing each atomic (in a branch
    // that holds nothing else), and every value that steers the loop is read
    // with readfirstlane.  (Lane-divergent loop conditions at the head and
    // the end of this loop let the compiler split it into separate loops for
    // lane 0 and the other lanes, which never meet at the barriers again.)
    // The compiler's atomic optimizer is off for this source: it rewrites a
    // returning atomic into a one-lane atomic followed by an immediate wait
    // and broadcast of the result, which would stall the claim below.
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const bool lane0 = (threadIdx.x & 63) == 0;
    uint32_t* const err = args.sync + kSyncStride * 8;
    uint32_t* const exits = err + 1;
    // With 8 queues a workgroup serves the queue of the XCD it runs on, so
    // that a queue's tiles, and hence its blocks' buffers, stay in one XCD's
    // L2 whatever the placement of workgroups on XCDs; the synchronisation
    // below relies on that.  A workgroup on an XCD beyond the eighth (none on
    // this part) serves no queue and stops the launch.
    const uint32_t xcc = __builtin_amdgcn_readfirstlane(hw_xcc_id());
    const bool serve = args.nq != 8 || xcc < 8;
    const int q = args.nq == 8 ? static_cast<int>(xcc & 7u) : 0;
    const bool local_sync = args.nq == 8;
    if (wave == 0 && lane0 && (args.inject || !serve))
        __hip_atomic_fetch_or(err, serve ? 1u : 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t qb = args.qbase[q], qlen = serve ? args.qbase[q + 1] - qb : 0u;
    uint32_t* prev_done = nullptr;    // counter of the item this workgroup finished last ...
    uint32_t prev_tiles = 0;          // ... and its tile count
    // Lowest NS iteration among the items this workgroup has read operands
    // for since its CU's L1 was last invalidated (the launch starts with it
    // invalidated).  Within a launch every buffer version belongs to one
    // iteration, and a block's versions are read in order, so the L1 can hold
    // a stale line for an item only if the item's iteration is above this.
    uint32_t t_low = 0xffffffffu;
    // The queue index of the next item is taken in the epilogue of an item's
    // last tile (by wave 0, once it has no load left to wait for), so that
    // the atomic's round trip (several microseconds under load) overlaps the
    // epilogue's stores; vector memory operations retire in order, so taken
    // any earlier it would stall the K loop's DMA waits.  A workgroup then
    // holds one item beyond the one it has finished computing, and takes
    // items in queue order, so the lowest unfinished item can always proceed.
    // The item descriptors are read from the LDS copy of the queue.
    uint32_t win0 = 0;
    {
        const uint32_t n0 = qlen < kLdsItems ? qlen : kLdsItems;
        for (uint32_t i = threadIdx.x; i < n0; i += blockDim.x) s_items[i] = args.items[qb + i];
    }
    uint32_t* const head = args.sync + kSyncStride * q;
    uint32_t idx_v = 0;      // the claimed index (lane 0 of wave 0), read once the stores have drained
    if (wave == 0 && lane0 && serve)
        idx_v = __hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    for (;;) {
        if (wave == 0) {
            // The previous tile's stores completed before the barrier that
            // ended it; the add publishes them.
            if (prev_done && lane0) {
                if (local_sync)
                    __hip_atomic_fetch_add(prev_done, prev_tiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else
                    __hip_atomic_fetch_add(prev_done, prev_tiles, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
            uint2 it = {kItemEnd, 0u};
            const uint32_t idx = __builtin_amdgcn_readfirstlane(idx_v);
            if (idx < qlen) {
                if (idx - win0 >= kLdsItems) {
                    // Only wave 0 reads the window; its LDS accesses complete in order.
                    win0 = idx;
                    const uint32_t n = qlen - win0 < kLdsItems ? qlen - win0 : kLdsItems;
                    for (uint32_t i = threadIdx.x; i < n; i += 64) s_items[i] = args.items[qb + win0 + i];
                }
                const uint2 raw = s_items[idx - win0];
                it.x = __builtin_amdgcn_readfirstlane(raw.x);
                it.y = __builtin_amdgcn_readfirstlane(raw.y);
                const uint32_t g = it.x & kBlockMask;
                int pi = 0;
                for (int i = 1; i < args.n; ++i)
                    if (g >= args.pr[i].first_blk) pi = i;
                const PersistProblem& pr = args.pr[pi];
                const uint32_t t = it.y >> 24, ph = (it.y >> 22) & 3u;
                const uint32_t need = t * (2 * pr.nsym + pr.nbx) + (ph >= 1 ? pr.nsym : 0u) + (ph >= 2 ? pr.nsym : 0u);
                uint32_t* const done = pr.done + kSyncStride * (g - pr.first_blk);
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                // The error word is read only while waiting: a workgroup whose
                // dependencies are met keeps going (the final check marks
                // every block left incomplete); with `inject` every workgroup
                // stops at its first item.
                for (;;) {
                    if (args.inject) {
                        it.x = kItemEnd;
                        break;
                    }
                    const uint32_t d = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                    if (d >= need) break;
                    const uint32_t e = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                    if (e != 0u) {
                        it.x = kItemEnd;
                        break;
                    }
                    if (__builtin_amdgcn_s_memrealtime() - t0 > args.spin_ticks) {
                        if (lane0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        it.x = kItemEnd;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // Acquire.  With XCD-local queues the XCD's L2 holds every
                // write to the block's buffers, so only this CU's L1 can be
                // stale, and only when t > t_low; the device-scope
                // invalidate drops its lines (a workgroup-scope one does not,
                // all of a workgroup's waves sharing one CU).  At device
                // scope the L2 can be stale too: always invalidate.
                if (!local_sync || t > t_low) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    t_low = t;
                } else {
                    t_low = t;    // t <= t_low here
                }
            }
            s_item = it;    // every lane of wave 0 writes the same value
        }
        __syncthreads();
        const uint2 raw = s_item;
        const uint32_t itx = __builtin_amdgcn_readfirstlane(raw.x), ity = __builtin_amdgcn_readfirstlane(raw.y);
        if (itx == kItemEnd) break;
        const uint32_t g = itx & kBlockMask;
        const int ntiles = static_cast<int>(itx >> 28) + 1;
        int pi = 0;
        for (int i = 1; i < args.n; ++i)
            if (g >= args.pr[i].first_blk) pi = i;
        const PersistProblem& pr = args.pr[pi];
        const int64_t blk = g - pr.first_blk;
        const int t = static_cast<int>(ity >> 24), ph = static_cast<int>((ity >> 22) & 3u);
        const int64_t xs = int64_t(pr.mp) * pr.np, as = int64_t(pr.mp) * pr.mp;
        const uint16_t* const xin = (t == 0 ? pr.x0 : pr.xb[t & 1]) + blk * xs;
        const uint16_t* const xin_lo = SPLIT ? pr.xlo[t & 1] + blk * xs : nullptr;
        // Tile c of the item (every tile of an item is of one product).
        const auto job = [&](int c) {
            int id = static_cast<int>(ity & 0x3fffffu) + c;
            TileJob j;
            j.p[1] = j.q[1] = nullptr;
            j.out[1] = nullptr;
            j.trace = t == 0 && pr.trace ? pr.trace + blk * pr.trace_stride : nullptr;
            j.ntrace = pr.mp / 32;
            if (ph < 2) {
                int r = 0, len = pr.mp / 256;
                while (id >= len) { id -= len; ++r; --len; }
                j.ti = r;
                j.tj = r + id;
            } else {
                j.ti = id % (pr.mp / 256);
                j.tj = id / (pr.mp / 256);
            }
            if (ph == 0) {
                j.p[0] = j.q[0] = xin;
                j.out[0] = pr.a + blk * as;
                j.p_bytes = j.q_bytes = static_cast<uint32_t>(xs * 2);
                j.K = pr.np;
                j.ldq = pr.np;
                j.ldo = pr.mp;
            } else if (ph == 1) {
                j.p[0] = j.q[0] = pr.a + blk * as;
                j.out[0] = pr.b + blk * as;
                if constexpr (SPLIT) j.out[1] = pr.blo + blk * as;
                j.p_bytes = j.q_bytes = static_cast<uint32_t>(as * 2);
                j.K = pr.mp;
                j.ldq = pr.mp;
                j.ldo = pr.mp;
            } else {
                j.p[0] = pr.b + blk * as;
                j.q[0] = xin;
                j.out[0] = (t + 1 == args.steps ? pr.xlast : pr.xb[(t + 1) & 1]) + blk * xs;
                j.p_bytes = static_cast<uint32_t>(as * 2);
                j.q_bytes = static_cast<uint32_t>(xs * 2);
                j.K = pr.mp;
                j.ldq = pr.np;
                j.ldo = pr.np;
                if constexpr (SPLIT) {
                    j.p[1] = pr.blo + blk * as;
                    j.q[1] = xin_lo;
                    j.out[1] = pr.xlo[(t + 1) & 1] + blk * xs;
                }
            }
            return j;
        };
        for (int c = 0; c < ntiles; ++c) {
            if (c > 0) __syncthreads();    // the previous tile's epilogue is done with LDS
            const bool last = c + 1 == ntiles;
            const auto claim = [&]() {
                if (wave == 0 && last && lane0)
                    idx_v = __hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            const TileJob j = job(c);
            if (ph == 0) {
                gemm_tile<kGram, 256, true, decltype(claim), !SPLIT>(j, lds, args.ca, args.cb, args.cc, args.eps, claim);
            } else if (ph == 1) {
                if constexpr (SPLIT)
                    gemm_tile<kPolySplit, 256, true, decltype(claim), false>(j, lds, args.ca, args.cb, args.cc, args.eps,
                                                                             claim);
                else
                    gemm_tile<kPoly, 256, true>(j, lds, args.ca, args.cb, args.cc, args.eps, claim);
            } else {
                if constexpr (SPLIT)
                    gemm_tile<kBxSplit, 256, true>(j, lds, args.ca, args.cb, args.cc, args.eps, claim);
                else
                    gemm_tile<kBx, 256, true>(j, lds, args.ca, args.cb, args.cc, args.eps, claim);
            }
        }
        // Every wave's stores (and wave 0's claim) complete before the barrier.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        prev_done = pr.done + kSyncStride * blk;
        prev_tiles = static_cast<uint32_t>(ntiles);
    }
    // Leave: the exit count tells the last workgroup out, which verifies the
    // run.  Every completion of this workgroup was published above, before
    // the item it found at the end.
    __shared__ uint32_t s_last;
    if (wave == 0) {
        uint32_t old = 0;
        if (lane0) old = __hip_atomic_fetch_add(exits, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        s_last = old + 1 == gridDim.x ? 1u : 0u;
    }
    __syncthreads();
    if (s_last) ns_loop_verify(args, err, lds);
}

// Prepares a loop launch: zeroes the counter regions (region r is [0, n[r])
// of p[r]) and copies the item list into the workspace from the library's
// pinned host copy.
struct SetupArgs {
    uint32_t* p[kMaxNsLoopProblems];
    uint32_t n[kMaxNsLoopProblems];
    int count;
    const uint2* src;         // host (pinned, device-readable)
    uint2* dst;               // workspace
    uint32_t items;
    uint32_t* status;         // null, or the call's two status words to clear
};

__global__ void k_loop_setup(SetupArgs z) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    for (int r = 0; r < z.count; ++r)
        if (i < z.n[r]) z.p[r][i] = 0u;
    if (i < z.items) z.dst[i] = z.src[i];
    if (z.status != nullptr && i < 2) z.status[i] = 0u;
}

// Every kernel instantiation is named explicitly: with implicit instantiation
// from the launchers below, hipcc emitted host launch stubs for only some of
// them, leaving undefined symbols in the shared library.
template __global__ void k_gemm<kGram, 64>(GemmArgs);
template __global__ void k_gemm<kPoly, 64>(GemmArgs);
template __global__ void k_gemm<kPolySplit, 64>(GemmArgs);
template __global__ void k_gemm<kBx, 64>(GemmArgs);
template __global__ void k_gemm<kBxSplit, 64>(GemmArgs);
template __global__ void k_gemm<kGram, 128>(GemmArgs);
template __global__ void k_gemm<kGram, 256>(GemmArgs);
template __global__ void k_gemm<kPoly, 128>(GemmArgs);
template __global__ void k_gemm<kPoly, 256>(GemmArgs);
template __global__ void k_gemm<kPolySplit, 128>(GemmArgs);
template __global__ void k_gemm<kPolySplit, 256>(GemmArgs);
template __global__ void k_gemm<kBx, 128>(GemmArgs);
template __global__ void k_gemm<kBx, 256>(GemmArgs);
template __global__ void k_gemm<kBxSplit, 128>(GemmArgs);
template __global__ void k_gemm<kBxSplit, 256>(GemmArgs);
template __global__ void k_ns_loop<false>(PersistArgs);
template __global__ void k_ns_loop<true>(PersistArgs);

}  // namespace

double& last_exec_flops() {
    thread_local double v = 0.0;
    return v;
}

namespace {

// Compute units of the current device (the rounds of the cost model below).
int64_t device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    return cus;
}

// Estimated cycles of one round of workgroups at reduction length K, from the
// measured per-K-step loop time and the prologue + epilogue of each tiling:
// a round is one 256-wide tile per CU, or two 128-wide tiles per CU (which
// share the CU; per flop the 128-wide tiling is about 1.3x slower: twice the
// operand traffic per MFMA).
// A 256-wide symmetric tile also stores its mirror (twice the bytes of a B'X
// tile), and when a launch is one round every workgroup stores at once, at
// the HBM limit: 25000 rather than 12000 fixed cycles (measured on the 124M
// attn Gram and polynomial, 240 tiles at K = 768, which run 1.8% faster per
// step as 128-wide tiles).
double round_cycles_big(int64_t K, bool sym) { return 1305.0 * double(K / 32) + (sym ? 25000.0 : 12000.0); }
double round_cycles_small(int64_t K) { return 812.0 * double(K / 32) + 8500.0; }
// 64-wide tiles: up to kTinyPerCU workgroups share a CU (32 KB of LDS each).
// A K step costs more per resident tile as the CU fills (LDS bandwidth: 4
// waves of 32 x 32 read twice the operand bytes per MFMA of the 64 x 64 wave
// tiles); measured per kind, cycles per K step with 1..5 tiles per CU.
constexpr int64_t kTinyPerCU = 5;
template <int KIND>
double tiny_step_cycles(int64_t per_cu) {
    static constexpr double gram[5] = {381, 510, 851, 1414, 1816};
    static constexpr double poly[5] = {373, 496, 664, 1218, 1419};
    static constexpr double poly_split[5] = {274, 371, 599, 911, 1477};
    static constexpr double bx[5] = {378, 552, 735, 1126, 1493};
    static constexpr double bx_split[5] = {585, 740, 835, 1162, 1494};    // per K step of the 3 K reduction
    const double* t = KIND == kGram ? gram : KIND == kPoly ? poly : KIND == kPolySplit ? poly_split
                    : KIND == kBx ? bx : bx_split;
    return t[per_cu - 1];
}
template <int KIND>
double tiny_cycles(int64_t tiles, int64_t K, int64_t cus) {
    const int64_t per_cu = (tiles + cus - 1) / cus;                 // tiles each CU runs in total
    const int64_t rounds = (per_cu + kTinyPerCU - 1) / kTinyPerCU;
    const int64_t last = per_cu - (rounds - 1) * kTinyPerCU;
    return 6500.0 + double(K / 32) * (double(rounds - 1) * tiny_step_cycles<KIND>(kTinyPerCU) +
                                      tiny_step_cycles<KIND>(last));
}

std::atomic<int> g_gemm_tiling{0};

// ---- automatic tiling
// The tilings give bitwise the same results but none of the estimates above
// ranks them reliably across shapes (the per-K-step cost depends on how many
// tiles share a CU, on L2 reuse and on the store traffic), so the choice is
// measured: per launch signature (kind, reduction length, device and every
// problem's padded sides and block count), the plans estimated within 2x of
// the best estimate each run kTileTrials launches timed with an event pair
// on the launch's stream, and once all those events have completed the plan
// with the lowest minimum time is kept.  Until then, and for launches that
// may not time (stream capture, the allocation-free entry point, more than
// kMaxTileKeys signatures), the best estimate is used.
constexpr int kTilePlans = 4;        // 64-wide, 128-wide, 256-wide, 256-wide with 128-wide quadrant tail
constexpr int kTileTrials = 3;
constexpr size_t kMaxTileKeys = 1024;
struct TileTune {
    int ncand = 0;
    int cand[kTilePlans] = {};
    int issued = 0;                                  // trial launches handed out
    int decided = -1;                                // the plan, or -1 while trials run
    hipEvent_t ev[kTilePlans * kTileTrials][2] = {};
    bool recorded[kTilePlans * kTileTrials] = {};
};
std::mutex g_tile_mu;
std::map<std::vector<int64_t>, TileTune> g_tile;     // under g_tile_mu (entries are never erased)
thread_local bool t_tile_no_trials = false;

struct TileChoice {
    int plan;
    TileTune* tune = nullptr;                        // set for a timed trial launch
    int trial = -1;
    bool started = false;
};

// Under g_tile_mu: decides once every trial's events have completed; false
// while some are pending.
bool tile_decide(TileTune& t, int fallback) {
    const int ntr = t.ncand * kTileTrials;
    for (int i = 0; i < ntr; ++i) {
        if (!t.recorded[i]) continue;
        const hipError_t q = hipEventQuery(t.ev[i][1]);
        if (q == hipErrorNotReady) return false;
        if (q != hipSuccess) t.recorded[i] = false;
    }
    float best[kTilePlans];
    for (float& b : best) b = -1.f;
    for (int i = 0; i < ntr; ++i) {
        float ms = 0.f;
        if (!t.recorded[i] || hipEventElapsedTime(&ms, t.ev[i][0], t.ev[i][1]) != hipSuccess) continue;
        float& b = best[i % t.ncand];
        if (b < 0.f || ms < b) b = ms;
    }
    t.decided = fallback;
    float win = -1.f;
    for (int c = 0; c < t.ncand; ++c)
        if (best[c] >= 0.f && (win < 0.f || best[c] < win)) {
            win = best[c];
            t.decided = t.cand[c];
        }
    for (auto& pair : t.ev)
        for (hipEvent_t& e : pair)
            if (e) {
                (void)hipEventDestroy(e);
                e = nullptr;
            }
    return true;
}

// est[p]: the plan's estimated cycles (kNever where it does not apply).
TileChoice tile_choose(const std::vector<int64_t>& key, const double (&est)[kTilePlans], hipStream_t s) {
    int model = 1;
    for (int p = 0; p < kTilePlans; ++p)
        if (est[p] < est[model]) model = p;
    TileChoice c{model};
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const bool can_time = !t_tile_no_trials && hipStreamIsCapturing(s, &cs) == hipSuccess &&
                          cs == hipStreamCaptureStatusNone;
    std::lock_guard<std::mutex> lock(g_tile_mu);
    auto it = g_tile.find(key);
    if (it == g_tile.end()) {
        if (!can_time || g_tile.size() >= kMaxTileKeys) return c;
        TileTune t;
        for (int p = 0; p < kTilePlans; ++p)
            if (est[p] <= 2.0 * est[model]) t.cand[t.ncand++] = p;
        if (t.ncand < 2) t.decided = model;
        it = g_tile.emplace(key, t).first;
    }
    TileTune& t = it->second;
    if (t.decided >= 0) {
        c.plan = t.decided;
        return c;
    }
    if (!can_time) return c;
    if (t.issued >= t.ncand * kTileTrials) {
        if (tile_decide(t, model)) c.plan = t.decided;
        return c;
    }
    const int i = t.issued;
    for (hipEvent_t& e : t.ev[i])
        if (!e && hipEventCreate(&e) != hipSuccess) return c;
    ++t.issued;
    c.plan = t.cand[i % t.ncand];
    c.tune = &t;
    c.trial = i;
    return c;
}

void tile_trial_start(TileChoice& c, hipStream_t s) {
    if (c.trial < 0) return;
    std::lock_guard<std::mutex> lock(g_tile_mu);
    c.started = hipEventRecord(c.tune->ev[c.trial][0], s) == hipSuccess;
}

void tile_trial_end(const TileChoice& c, hipStream_t s) {
    if (c.trial < 0 || !c.started) return;
    std::lock_guard<std::mutex> lock(g_tile_mu);
    if (hipEventRecord(c.tune->ev[c.trial][1], s) == hipSuccess) c.tune->recorded[c.trial] = true;
}

// Tiling of one launch (n products of one kind): the width set with
// set_gemm_tiling where the shapes allow it, else by the automatic choice
// above among four plans, estimated over all their tiles together:
//  * 64-wide tiles throughout (up to 1024 per round);
//  * 128-wide tiles throughout (512 per round);
//  * 256-wide tiles (256 per round) with the last partial round split into
//    128-wide quadrants in a second launch;
//  * 256-wide tiles throughout, the last round partial.
// The products share the reduction length K (the caller groups them so).
template <int KIND>
hipError_t run(const Plan* const* plans, GemmArgs a, hipStream_t s) {
    constexpr bool SYM = KIND == kGram || KIND == kPoly || KIND == kPolySplit;
    const int64_t K = a.pr[0].K;
    // the split B X runs a reduction three times as long (Bh Xh, Bh Xl, Bl Xh)
    const int64_t Kc = KIND == kBxSplit ? 3 * K : K;
    auto geometry = [&](int bt) {
        int64_t first = 0;
        for (int i = 0; i < a.n; ++i) {
            GemmProblem& g = a.pr[i];
            const Plan& p = *plans[i];
            if (SYM) {
                g.T = static_cast<int>(p.mp / bt);
                g.tiles = static_cast<uint32_t>(g.T * (g.T + 1) / 2);
            } else {
                g.tiles_i = static_cast<uint32_t>(p.mp / bt);
                g.tiles = g.tiles_i * static_cast<uint32_t>(p.np / bt);
            }
            g.first = static_cast<uint32_t>(first);
            first += int64_t(g.tiles) * p.nb;
            if (first > 0x3fffffffLL) return int64_t(-1);
        }
        return first;
    };
    // Executed MFMA flops of the launches (for the timing diagnostics): every
    // workgroup computes a bt x bt tile over the reduction, except the lower
    // quadrants of diagonal 256-wide tiles in quadrant mode, which return,
    // and diagonal 256-wide tiles, which compute 10 of their 16 64 x 64 blocks.
    auto launch = [&](int bt, int64_t total, uint32_t quad, uint32_t base) {
        a.quad = quad;
        a.big_base = base;
        a.total = static_cast<uint32_t>(total);
        double tiles = double(total);
        if (SYM && bt == 256 && !quad) {
            for (int64_t t = 0; t < total; ++t) {
                int pi = 0;
                for (int i = 1; i < a.n; ++i)
                    if (t >= int64_t(a.pr[i].first)) pi = i;
                int id = static_cast<int>((t - a.pr[pi].first) % a.pr[pi].tiles), len = a.pr[pi].T;
                while (id > 0 && id >= len) { id -= len; --len; }
                if (id == 0) tiles -= 0.375;    // the row's diagonal tile
            }
        }
        if (quad && SYM) {
            tiles = 0;
            for (int64_t t = base; t < int64_t(base) + total / 4; ++t) {
                int pi = 0;
                for (int i = 1; i < a.n; ++i)
                    if (t >= int64_t(a.pr[i].first)) pi = i;
                int id = static_cast<int>((t - a.pr[pi].first) % a.pr[pi].tiles), len = a.pr[pi].T, r = 0;
                while (id >= len) { id -= len; ++r; --len; }
                tiles += id == 0 ? 3 : 4;     // id == 0: the row's diagonal tile
            }
        }
        last_exec_flops() += tiles * 2.0 * double(bt) * double(bt) * double(Kc);
        if (bt == 256) {
            k_gemm<KIND, 256><<<dim3(a.total), dim3(tile_threads<256>()), 0, s>>>(a);
        } else if (bt == 128) {
            k_gemm<KIND, 128><<<dim3(a.total), dim3(tile_threads<128>()), 0, s>>>(a);
        } else {
            k_gemm<KIND, 64><<<dim3(a.total), dim3(tile_threads<64>()), 0, s>>>(a);
        }
        return hipGetLastError();
    };
    const int64_t kCUs = device_cus();
    bool big_ok = true;
    for (int i = 0; i < a.n; ++i) {
        if (a.pr[i].K != K) return hipErrorInvalidValue;
        big_ok = big_ok && plans[i]->mp % 256 == 0 && (SYM || plans[i]->np % 256 == 0);
    }
    constexpr double kNever = 1e300;
    const int64_t small = geometry(128);
    if (small < 0) return hipErrorInvalidValue;
    const double t_small = double((small + 2 * kCUs - 1) / (2 * kCUs)) * round_cycles_small(Kc);
    const int64_t tiny = geometry(64);      // negative past the tile index range
    const double t_tiny = tiny < 0 ? kNever : tiny_cycles<KIND>(tiny, Kc, kCUs);
    int64_t big = 0, full = 0, tail = 0;
    double t_big = kNever, t_split = kNever;
    if (big_ok) {
        big = geometry(256);
        full = big / kCUs;
        tail = big % kCUs;
        const double rb = round_cycles_big(Kc, SYM);
        t_split = double(full) * rb + double((4 * tail + 2 * kCUs - 1) / (2 * kCUs)) * round_cycles_small(Kc);
        t_big = double(full + (tail ? 1 : 0)) * rb;
    }
    // plan: 0 = 64-wide, 1 = 128-wide, 2 = 256-wide, 3 = 256-wide with 128-wide quadrants for the tail
    TileChoice ch{1};
    const int force = g_gemm_tiling.load();
    if (force == 64 && tiny >= 0) {
        ch.plan = 0;
    } else if (force == 128 || (force == 256 && !big_ok)) {
        ch.plan = 1;
    } else if (force == 256) {
        ch.plan = 2;
    } else {
        // the split plan is distinct only with both full rounds and a tail
        const double est[kTilePlans] = {t_tiny, t_small, t_big, full > 0 && tail > 0 ? t_split : kNever};
        std::vector<int64_t> key = {KIND, Kc, device_cus(), a.n};
        for (int i = 0; i < a.n; ++i) {
            key.push_back(plans[i]->mp);
            key.push_back(plans[i]->np);
            key.push_back(plans[i]->nb);
        }
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess) key.push_back(dev);
        ch = tile_choose(key, est, s);
    }
    tile_trial_start(ch, s);
    hipError_t e = hipSuccess;
    switch (ch.plan) {
        case 0:
            geometry(64);
            e = launch(64, tiny, 0, 0);
            break;
        case 2:
            geometry(256);
            e = launch(256, big, 0, 0);
            break;
        case 3:
            geometry(256);
            if (full > 0) e = launch(256, full * kCUs, 0, 0);
            if (e == hipSuccess && tail > 0) e = launch(128, 4 * tail, 1, static_cast<uint32_t>(full * kCUs));
            break;
        default:
            geometry(128);
            e = launch(128, small, 0, 0);
            break;
    }
    tile_trial_end(ch, s);
    return e;
}

}  // namespace

hipError_t launch_gram(const GramOp* ops, int n, uint32_t* status, hipStream_t s) {
    if (n < 1 || n > kMaxProblems) return hipErrorInvalidValue;
    GemmArgs a{};
    const Plan* plans[kMaxProblems];
    a.n = n;
    a.status = status;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *ops[i].plan;
        GemmProblem& g = a.pr[i];
        plans[i] = &p;
        g.p[0] = ops[i].x;
        g.q[0] = ops[i].x;
        g.out[0] = ops[i].a;
        g.trace = ops[i].trace;
        g.trace_stride = p.trace_stride;
        g.ntrace = static_cast<int>(p.mp / 32);
        g.p_stride = g.q_stride = p.mp * p.np;
        g.out_stride = p.mp * p.mp;
        g.K = p.np;
        g.ldo = p.mp;
        g.p_bytes = g.q_bytes = static_cast<uint32_t>(p.mp * p.np * 2);
    }
    return run<kGram>(plans, a, s);
}

hipError_t launch_poly(const PolyOp* ops, int n, float ca, float cb, float cc, float eps, hipStream_t s) {
    if (n < 1 || n > kMaxProblems) return hipErrorInvalidValue;
    GemmArgs a{};
    const Plan* plans[kMaxProblems];
    a.n = n;
    a.ca = ca;
    a.cb = cb;
    a.cc = cc;
    a.eps = eps;
    const bool split = ops[0].b_lo != nullptr;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *ops[i].plan;
        GemmProblem& g = a.pr[i];
        if ((ops[i].b_lo != nullptr) != split) return hipErrorInvalidValue;
        plans[i] = &p;
        g.p[0] = ops[i].a;
        g.q[0] = ops[i].a;
        g.out[0] = ops[i].b_hi;
        g.out[1] = ops[i].b_lo;
        g.trace = const_cast<float*>(ops[i].trace);
        g.trace_stride = p.trace_stride;
        g.ntrace = static_cast<int>(p.mp / 32);
        g.p_stride = g.q_stride = p.mp * p.mp;
        g.out_stride = p.mp * p.mp;
        g.K = p.mp;
        g.ldq = p.mp;
        g.ldo = p.mp;
        g.p_bytes = g.q_bytes = static_cast<uint32_t>(p.mp * p.mp * 2);
    }
    return split ? run<kPolySplit>(plans, a, s) : run<kPoly>(plans, a, s);
}

hipError_t launch_bx(const BxOp* ops, int n, float eps, hipStream_t s) {
    if (n < 1 || n > kMaxProblems) return hipErrorInvalidValue;
    GemmArgs a{};
    const Plan* plans[kMaxProblems];
    a.n = n;
    a.eps = eps;
    const bool split = ops[0].b_lo != nullptr;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *ops[i].plan;
        GemmProblem& g = a.pr[i];
        if ((ops[i].b_lo != nullptr) != split) return hipErrorInvalidValue;
        plans[i] = &p;
        g.p[0] = ops[i].b_hi;
        g.p[1] = ops[i].b_lo;
        g.q[0] = ops[i].x_hi;
        g.q[1] = ops[i].x_lo;
        g.out[0] = ops[i].out_hi;
        g.out[1] = ops[i].out_lo;
        g.trace = const_cast<float*>(ops[i].trace);
        g.trace_stride = p.trace_stride;
        g.ntrace = static_cast<int>(p.mp / 32);
        g.p_stride = p.mp * p.mp;
        g.q_stride = p.mp * p.np;
        g.out_stride = p.mp * p.np;
        g.K = p.mp;
        g.ldq = p.np;
        g.ldo = p.np;
        g.p_bytes = static_cast<uint32_t>(p.mp * p.mp * 2);
        g.q_bytes = static_cast<uint32_t>(p.mp * p.np * 2);
    }
    return split ? run<kBxSplit>(plans, a, s) : run<kBx>(plans, a, s);
}

hipError_t launch_gram(const Plan& p, const uint16_t* x, uint16_t* a_out, float* trace, uint32_t* status,
                       hipStream_t s) {
    const GramOp op{&p, x, a_out, trace};
    return launch_gram(&op, 1, status, s);
}

hipError_t launch_poly(const Plan& p, const uint16_t* a_in, uint16_t* b_hi, uint16_t* b_lo, float ca, float cb,
                       float cc, const float* trace, float eps, hipStream_t s) {
    const PolyOp op{&p, a_in, b_hi, b_lo, trace};
    return launch_poly(&op, 1, ca, cb, cc, eps, s);
}

hipError_t launch_bx(const Plan& p, const uint16_t* b_hi, const uint16_t* b_lo, const uint16_t* x_hi,
                     const uint16_t* x_lo, uint16_t* out_hi, uint16_t* out_lo, const float* trace, float eps,
                     hipStream_t s) {
    const BxOp op{&p, b_hi, b_lo, x_hi, x_lo, out_hi, out_lo, trace};
    return launch_bx(&op, 1, eps, s);
}

// ---------------------------------------------------------------- persistent NS loop (host)
namespace {

std::atomic<int> g_ns_mode{0};
std::atomic<int> g_loop_fault{0};

// One distinct set of block shapes: its queues, built once by the host list
// scheduler and kept in pinned host memory (never device memory), from which
// every launch copies them into the caller's workspace on the caller's stream.
struct Schedule {
    uint2* host_items = nullptr;   // hipHostMalloc, device-readable, kept until the process ends
    uint32_t count = 0;
    uint32_t qbase[9] = {};
    int nq = 1;
};

constexpr size_t kMaxSchedules = 64;
constexpr uint64_t kMaxItems = uint64_t(1) << 22;
std::mutex g_sched_mu;
std::map<std::vector<int64_t>, Schedule> g_sched;

// The queues of one set of shapes (host only).  With 8 queues every
// workgroup serves the queue of the XCD it runs on, so the cost model prices
// the XCD-local synchronisation.
hipError_t build_schedule(const std::vector<LoopDims>& dims, const std::vector<int64_t>& nbs, int steps, int workers,
                          Schedule& out) {
    std::vector<ScheduleItem> items;
    schedule_items(dims, nbs, steps, workers, true, items, out.qbase, out.nq);
    static_assert(sizeof(ScheduleItem) == sizeof(uint2), "item layout");
    out.count = static_cast<uint32_t>(items.size());
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&out.host_items), std::max<size_t>(1, items.size()) * sizeof(uint2),
                                 hipHostMallocDefault);
    if (e != hipSuccess) {
        out.host_items = nullptr;
        return e;
    }
    if (!items.empty()) std::memcpy(out.host_items, items.data(), items.size() * sizeof(uint2));
    return hipSuccess;
}

}  // namespace

void set_ns_schedule(int mode) { g_ns_mode.store(mode); }
void set_loop_fault(int mode) { g_loop_fault.store(mode); }
void set_gemm_tiling(int width) { g_gemm_tiling.store(width); }
TileTrialsOff::TileTrialsOff() : prev_(t_tile_no_trials) { t_tile_no_trials = true; }
TileTrialsOff::~TileTrialsOff() { t_tile_no_trials = prev_; }

// Cache key of a schedule: device, steps, workgroups, then (mp, np, nb) per problem.
std::vector<int64_t> schedule_key(const NsLoopProblem* probs, int n, int ns_steps, int dev, int cus) {
    std::vector<int64_t> key{dev, ns_steps, cus};
    for (int i = 0; i < n; ++i) key.insert(key.end(), {probs[i].plan->mp, probs[i].plan->np, probs[i].plan->nb});
    return key;
}

uint64_t ns_loop_items_cap(const Plan* const* plans, int n, int ns_steps) {
    if (n < 1 || n > kMaxNsLoopProblems || ns_steps < 1 || ns_steps > 255) return 0;
    uint64_t items = 0, blocks = 0;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *plans[i];
        if (p.small || p.precision != plans[0]->precision || p.nb < 1 || p.mp % 256 || p.np % 256) return 0;
        const uint64_t T = uint64_t(p.mp / 256), Tn = uint64_t(p.np / 256);
        if (T * Tn >= (uint64_t(1) << 22)) return 0;
        // at most one item per tile: T (T + 1) / 2 tiles per symmetric product, T Tn for B X
        items += uint64_t(p.nb) * uint64_t(ns_steps) * (T * (T + 1) + T * Tn);
        blocks += uint64_t(p.nb);
    }
    return items <= kMaxItems && blocks < (uint64_t(1) << 27) ? items : 0;
}

bool ns_loop_eligible(const NsLoopProblem* probs, int n, int ns_steps) {
    if (n < 1 || n > kMaxNsLoopProblems) return false;
    const Plan* plans[kMaxNsLoopProblems];
    for (int i = 0; i < n; ++i) plans[i] = probs[i].plan;
    return ns_loop_items_cap(plans, n, ns_steps) > 0;
}

namespace {

// Automatic choice (schedule mode 0), per set of shapes: the first
// kTrialCalls calls alternate the per-product launches (even calls) and the
// persistent loop (odd calls), each timed with an event pair on the call's
// stream; once the last trial's events have completed, the schedule with the
// lower minimum time over the trials after the first of each is kept (the
// minimum discounts calls slowed by other work).  Both schedules give bitwise
// the same results.
constexpr int kTrialCalls = 10;
constexpr size_t kMaxAutoSets = 256;
struct AutoState {
    int calls = 0;
    int decided = -1;                        // -1 pending, 0 per-product, 1 persistent
    hipEvent_t ev[kTrialCalls][2] = {};
    bool started[kTrialCalls] = {};
    bool recorded[kTrialCalls] = {};
};
std::map<std::vector<int64_t>, AutoState> g_auto;    // under g_sched_mu

void release_events(AutoState& st) {
    for (auto& pair : st.ev)
        for (hipEvent_t& e : pair)
            if (e) {
                (void)hipEventDestroy(e);
                e = nullptr;
            }
}

// The cached schedule of this set of shapes, built on first use (not under
// stream capture: building allocates pinned host memory); null when the
// cache is full, building failed or was not allowed (the caller then runs per
// product).
const Schedule* find_schedule(const NsLoopProblem* probs, int n, int ns_steps, int dev, int cus, bool may_build) {
    const std::vector<int64_t> key = schedule_key(probs, n, ns_steps, dev, cus);
    auto it = g_sched.find(key);
    if (it != g_sched.end()) return &it->second;
    if (!may_build || g_sched.size() >= kMaxSchedules) return nullptr;
    std::vector<LoopDims> dims;
    std::vector<int64_t> nbs;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *probs[i].plan;
        const uint32_t T = uint32_t(p.mp / 256), Tn = uint32_t(p.np / 256);
        dims.push_back({int(p.mp), int(p.np), T * (T + 1) / 2, T * Tn, p.precision == MUON_PRECISION_ACCURATE});
        nbs.push_back(p.nb);
    }
    Schedule sc;
    if (build_schedule(dims, nbs, ns_steps, cus, sc) != hipSuccess) return nullptr;
    return &g_sched.emplace(key, sc).first->second;
}

}  // namespace

NsChoice ns_schedule_begin(const NsLoopProblem* probs, int n, int ns_steps, hipStream_t s) {
    NsChoice c;
    const int mode = g_ns_mode.load();
    if (mode == 1 || !ns_loop_eligible(probs, n, ns_steps)) return c;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return c;
    // Under stream capture nothing is allocated or timed: a settled choice
    // (and the queue it needs) is reused, anything else runs per product.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const bool capturing = hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
    std::lock_guard<std::mutex> lock(g_sched_mu);
    // The loop needs its queue: without one (cache full, no pinned host
    // memory, or capture) the call runs per product, which gives the same
    // results.
    const Schedule* sched = find_schedule(probs, n, ns_steps, dev, cus, !capturing);
    if (sched == nullptr) return c;
    c.sched = sched;
    c.cus = cus;
    if (mode == 2) {
        c.persistent = true;
        return c;
    }
    const std::vector<int64_t> key = schedule_key(probs, n, ns_steps, dev, cus);
    auto it = g_auto.find(key);
    if (capturing) {
        c.persistent = it != g_auto.end() && it->second.decided == 1;
        return c;
    }
    if (it == g_auto.end()) {
        if (g_auto.size() >= kMaxAutoSets) return c;
        it = g_auto.emplace(key, AutoState()).first;
    }
    AutoState& st = it->second;
    if (st.decided >= 0) {
        c.persistent = st.decided == 1;
        return c;
    }
    if (st.calls >= kTrialCalls) {
        // decide once every trial's events have completed
        bool ready = true, failed = false;
        for (int i = 0; i < kTrialCalls && ready; ++i) {
            failed = failed || !st.recorded[i];
            ready = !st.recorded[i] || hipEventQuery(st.ev[i][1]) == hipSuccess;
        }
        if (ready && failed) {
            // a trial was not timed (event record failed): keep per-product
            st.decided = 0;
            release_events(st);
            return c;
        }
        if (ready) {
            float best[2] = {0.f, 0.f};
            bool ok = true;
            for (int i = 2; i < kTrialCalls; ++i) {
                float ms = 0.f;
                ok = ok && hipEventElapsedTime(&ms, st.ev[i][0], st.ev[i][1]) == hipSuccess;
                if (ok && (best[i & 1] == 0.f || ms < best[i & 1])) best[i & 1] = ms;
            }
            st.decided = ok && best[1] > 0.f && best[1] < best[0] ? 1 : 0;
            release_events(st);
            c.persistent = st.decided == 1;
            return c;
        }
        c.persistent = (st.calls++ & 1) != 0;   // keep alternating, untimed, until then
        return c;
    }
    const int i = st.calls;
    for (hipEvent_t& e : st.ev[i])
        if (!e && hipEventCreate(&e) != hipSuccess) return c;
    ++st.calls;
    c.persistent = (i & 1) != 0;
    c.trial = i;
    c.key = &it->first;
    return c;
}

void ns_schedule_start(const NsChoice& c, hipStream_t s) {
    if (c.trial < 0) return;
    std::lock_guard<std::mutex> lock(g_sched_mu);
    auto it = g_auto.find(*c.key);
    if (it == g_auto.end() || it->second.decided >= 0) return;
    AutoState& st = it->second;
    st.started[c.trial] = hipEventRecord(st.ev[c.trial][0], s) == hipSuccess;
}

void ns_schedule_end(const NsChoice& c, hipStream_t s) {
    if (c.trial < 0) return;
    std::lock_guard<std::mutex> lock(g_sched_mu);
    auto it = g_auto.find(*c.key);
    if (it == g_auto.end() || it->second.decided >= 0) return;
    AutoState& st = it->second;
    if (st.started[c.trial] && hipEventRecord(st.ev[c.trial][1], s) == hipSuccess) st.recorded[c.trial] = true;
}

size_t ns_loop_sync_bytes(int64_t total_blocks) {
    return (size_t(kSyncLines + total_blocks) * kSyncStride * 4 + 255) & ~size_t(255);
}

hipError_t launch_ns_loop(const NsLoopProblem* probs, int n, int ns_steps, float ca, float cb, float cc, float eps,
                          const NsChoice& choice, uint2* items_ws, uint64_t items_cap, uint32_t* status,
                          bool clear_status, hipStream_t s) {
    if (!choice.persistent || choice.sched == nullptr || !ns_loop_eligible(probs, n, ns_steps) || status == nullptr)
        return hipErrorInvalidValue;
    const Schedule& sc = *static_cast<const Schedule*>(choice.sched);
    if (items_ws == nullptr || sc.count > items_cap) return hipErrorInvalidValue;
    for (int i = 0; i < n; ++i)
        if (probs[i].sync == nullptr) return hipErrorInvalidValue;
    PersistArgs a{};
    a.n = n;
    a.steps = ns_steps;
    a.ca = ca;
    a.cb = cb;
    a.cc = cc;
    a.eps = eps;
    a.sync = probs[0].sync;
    a.status = status;
    const int fault = g_loop_fault.load();
    a.inject = fault == 1 ? 1 : 0;
    a.spin_ticks = fault == 2 ? 0 : 100000000ull;   // 1 s of the 100 MHz real-time counter
    SetupArgs z{};
    z.count = n;
    uint32_t zmax = 0;
    uint32_t first = 0;
    const bool split = probs[0].plan->precision == MUON_PRECISION_ACCURATE;
    for (int i = 0; i < n; ++i) {
        const Plan& p = *probs[i].plan;
        const uint32_t T = uint32_t(p.mp / 256), Tn = uint32_t(p.np / 256);
        PersistProblem& pr = a.pr[i];
        pr.x0 = probs[i].x0;
        pr.xb[0] = probs[i].x[0];
        pr.xb[1] = probs[i].x[1];
        pr.xlast = probs[i].xlast;
        pr.xlo[0] = probs[i].xlo[0];
        pr.xlo[1] = probs[i].xlo[1];
        pr.a = probs[i].a;
        pr.b = probs[i].b;
        pr.blo = probs[i].blo;
        if (split != (probs[i].blo != nullptr && probs[i].xlo[0] != nullptr && probs[i].xlo[1] != nullptr))
            return hipErrorInvalidValue;
        pr.trace = probs[i].trace;
        pr.trace_stride = p.trace_stride;
        pr.done = probs[i].sync + kSyncLines * kSyncStride;
        z.p[i] = probs[i].sync;
        z.n[i] = uint32_t((kSyncLines + p.nb) * kSyncStride);
        zmax = std::max(zmax, z.n[i]);
        pr.mp = int32_t(p.mp);
        pr.np = int32_t(p.np);
        pr.first_blk = first;
        pr.nb = uint32_t(p.nb);
        pr.nsym = T * (T + 1) / 2;
        pr.nbx = T * Tn;
        first += uint32_t(p.nb);
    }
    a.items = items_ws;
    a.nq = sc.nq;
    for (int q = 0; q < 9; ++q) a.qbase[q] = sc.qbase[q];
    z.src = sc.host_items;
    z.dst = items_ws;
    z.items = sc.count;
    z.status = clear_status ? status : nullptr;
    const uint32_t work = std::max(std::max(zmax, sc.count), 2u);
    k_loop_setup<<<dim3((work + 255) / 256), dim3(256), 0, s>>>(z);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    double ex = 0.0;
    for (int i = 0; i < n; ++i) {
        const PersistProblem& pr = a.pr[i];
        // diagonal tiles of the symmetric products compute 10 of 16 64 x 64 blocks
        const double sym = double(pr.nsym) - 0.375 * double(pr.mp / 256);
        ex += double(pr.nb) * double(ns_steps) * 2.0 * 256.0 * 256.0 *
              (sym * pr.np + sym * pr.mp + double(pr.nbx) * pr.mp * (split ? 3.0 : 1.0));
    }
    last_exec_flops() += ex;
    if (split)
        k_ns_loop<true><<<dim3(choice.cus), dim3(tile_threads<256>()), 0, s>>>(a);
    else
        k_ns_loop<false><<<dim3(choice.cus), dim3(tile_threads<256>()), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace muon
