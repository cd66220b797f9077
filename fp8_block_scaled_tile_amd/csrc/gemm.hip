// gemm.hip -- block-scaled FP8 GEMM on gfx950 FP8 MFMA.
//
// The main linear-layer GEMMs of the recipe run on FP8 with fine-grained
// block scales (arXiv report "Puro-2B" section 2.1; training.farm blog
// section "FP8").  Every operand is E4M3 codes with one FP32 scale per
// 128-deep K-block of each row (activations) or per 128x128 block (weights),
// so the product is
//     C[m][n] = sum_kb sA(kb, m) * sB(kb, n) * P_kb[m][n],
//     P_kb    = sum over the 128 k of block kb of dec(a[m][k]) * dec(b[n][k]).
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KB LDS per CU):
//  * One workgroup = 512 threads (8 waves, 2 per SIMD) computes a 256x256
//    tile of C.  Each K-step is exactly one scale block (128 deep): A and B
//    slices of 256x128 bytes are staged in LDS, double buffered (128 KB).
//  * Each wave owns a 128(M) x 64(N) sub-tile as 8x4 MFMA tiles of 16x16.
//    One v_mfma_f32_16x16x128_f8f6f4 covers a whole K-block, so the partial
//    product P_kb of a 16x16 tile comes out of a single instruction and is
//    folded into the FP32 accumulator with one FMA per element:
//        acc = fma(P_kb, sA*sB, acc).
//  * FWD / DGRAD issue the MFMA with the B-side fragment as its first
//    operand, so each lane's 4 accumulator rows are 4 consecutive n of one
//    m: the A-side scale sA(kb, m) is one value per lane per tile, and sB is
//    constant over the wave's 64 columns (they sit inside one 128-wide
//    weight block).  WGRAD's sB varies per column; it issues the A-side
//    fragment first and pays one extra multiply per element.
//  * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled per
//    row (swz for A and WGRAD's B, swz_b for FWD / DGRAD's B); fragment
//    reads (16 rows x 32 bytes per instruction group) and the staging
//    writes are then bank-conflict free.
//  * Persistent launch: one workgroup per CU walks its (split, tile) units;
//    the next unit's first K-block is staged during the last one, and a
//    finished unit's epilogue runs under the next block's MFMAs.  Unit ids
//    are remapped so the 32 tiles that run together on one XCD form a
//    compact 4(M) x 8(N) group sharing that XCD's L2.
//  * bf16 output leaves as stores of 64 contiguous bytes per row and
//    instruction: non-temporal in the row layouts, so the streamed output
//    does not evict the A / B panels that the other workgroups re-read;
//    ordinary in the [K][N] layouts, where non-temporal ones cost time and
//    extra write-back (measured).
//  * Small-output problems split K across workgroups; the FP32 partials go
//    to the caller's workspace and a second kernel sums them in a fixed
//    order (deterministic).
#include "device_common.hpp"
#include "launch.hpp"

#include <mutex>

namespace puro {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int NTHREADS = 512;
constexpr int WM = 128;              // wave tile rows (M)
constexpr int WN = 64;               // wave tile cols (N)
constexpr int TM = WM / 16;          // 8 MFMA tiles along M
constexpr int TN = WN / 16;          // 4 MFMA tiles along N
constexpr int TILE_BYTES = BM * BK;  // 32 KB per operand slice
// Tiles per group along M in the unit order.  The 32 tiles that run together
// on one XCD cover 4 M-tiles x 8 N-tiles; the 4 A panels stay in use for the
// whole group and (at K = 2048, 512 KB each) fit in the XCD's L2 beside the
// streamed B panels.  Measured 1-3% faster than 8 on the block GEMMs.
constexpr int GROUP_M = 4;

// MODE_BF16 is the BF16 comparator: C = A . B^T on bf16 operands with the
// same tiling, staging and schedule, no block scales.  K is passed in bytes
// (2 per element), so a 128-byte K-block holds 64 bf16 values.
// MODE_DGRAD_W is DGRAD with B read straight from the weight's codes
// W [K = out][N = in] (N-contiguous) instead of their transposed copy: the
// K-block's 128 weight rows are staged as they lie and the B fragments are
// read with the gfx950 LDS transpose read (ds_read_b64_tr_b8).  MODE_FWD_T
// is FWD the same way, with B the transposed weight codes W^T [K = in][N =
// out] and the FWD scale indexing.
enum { MODE_FWD = 0, MODE_DGRAD = 1, MODE_WGRAD = 2, MODE_BF16 = 3, MODE_DGRAD_W = 4,
       MODE_FWD_T = 5 };
// B staged as [K][N] rows and read with transpose reads
constexpr bool b_kn(int mode) { return mode == MODE_DGRAD_W || mode == MODE_FWD_T; }
enum { OUT_BF16 = 0, OUT_FP32 = 1, OUT_FP32_ACC = 2, OUT_PARTIAL = 3 };

// LDS rows are 128 bytes (one K-block of one row).  The 16-byte chunk c of
// row r is stored at chunk position c ^ (r & 7) ^ ((r >> 3) & 1): a fragment
// read (16 consecutive rows, one chunk each per 16-lane phase) and the
// staging writes (8 chunks of 2 consecutive rows per phase) then touch 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// FWD / DGRAD read their B slice in a permuted row order (see frag_off_b):
// fragment lane i reads row r = 8*(i>>2) + (i&3) (+ 4, 32 or 36 for tiles
// 1-3).  Its swizzle is the A swizzle of the lane index, written in the row
// bits that carry it (bits 0, 1, 3, 4; bits 2 and 5 only select the tile):
// position = c ^ swz(i).  Lanes 0-7 and 8-15 of every phase then hit 8
// distinct 16-byte bank groups each, and the 16 lanes of a phase 16 distinct
// ones, like the A reads.  (Masks built from row bits 1, 3 and 4 alone left
// pairs of lanes 0-7 on one group: 2-way conflicts, 0.28 conflict cycles per
// LDS access in the counters.)  The staging writes are linear in LDS, so any
// per-row XOR keeps them conflict-free.
__device__ __forceinline__ int swz_b(int row)
{
    return ((row & 3) | (((row >> 3) & 1) << 2)) ^ ((row >> 4) & 1);
}
template <int MODE>
__device__ __forceinline__ int swz_stage_b(int row) { return MODE == 2 ? swz(row) : swz_b(row); }

// 32-byte MFMA operand fragment of a 16x128 slice whose first row is a
// multiple of 16: lane l holds row (l & 15) of the slice, logical chunks
// 2*(l>>4) and 2*(l>>4)+1.  The swizzle of a row depends only on its low 4
// bits, i.e. on the lane, so each lane's two byte offsets within any slice
// are fixed (FragOff) and the slice base folds into the instruction's
// immediate offset.  The A-side and B-side fragments use the same
// k <-> (lane, byte) mapping, so every product pairs a[m][k] with b[n][k]
// whatever order the hardware sums in.
struct FragOff {
    int lo, hi;
};

__device__ __forceinline__ FragOff frag_off(int lane)
{
    const int r = lane & 15;
    const int c0 = 2 * (lane >> 4);
    return {r * BK + ((c0 ^ swz(r)) << 4), r * BK + (((c0 + 1) ^ swz(r)) << 4)};
}

// B-side fragments of FWD / DGRAD: fragment row i of MFMA tile tn is B row
// 8*(i>>2) + (i&3) + 4*(tn&1) + 32*(tn>>1) of the wave's 64, so the lanes
// with (lane >> 4) == g hold output columns 8*g .. 8*g+7 (tiles 0, 1) and
// 32+8*g .. 32+8*g+7 (tiles 2, 3).  One 16-byte bf16 store per lane then
// covers 64 contiguous bytes of a row across the 4 lane groups.  The row's
// swizzle mask does not depend on tn (it uses row bits 0, 1, 3, 4), so tile tn
// is the tn = 0 offsets plus b_tile_rows(tn) rows.
__device__ __forceinline__ int b_tile_rows(int tn) { return 4 * (tn & 1) + 32 * (tn >> 1); }

__device__ __forceinline__ FragOff frag_off_b(int lane)
{
    const int i = lane & 15;
    const int r = 8 * (i >> 2) + (i & 3);
    const int c0 = 2 * (lane >> 4);
    return {r * BK + ((c0 ^ swz_b(r)) << 4), r * BK + (((c0 + 1) ^ swz_b(r)) << 4)};
}

// [K][N] modes (DGRAD_W, FWD_T): the staged B slice is 128 rows (k) of 256 bytes (the
// tile's 256 columns n).  The 16-byte unit u of row r is stored at unit
// position u ^ swz_w(r).  A transpose read (below) has its 32 lanes of one
// pass read one 16-byte unit in each of 16 rows r = 32*g + 8*j + m (g = 0, 1;
// m = 0..7); the mask gives those 16 rows 16 distinct unit positions, so the
// pass touches every bank once.  The staging copies are linear in LDS.
__device__ __forceinline__ int swz_w(int row) { return (row & 7) | (((row >> 5) & 1) << 3); }

// ds_read_b64_tr_b8 on gfx950 (measured): within each 16-lane group, input
// lane 2*m + p supplies an 8-byte chunk and output lane t receives byte
// (t & 7) of the chunks of input lanes (t >> 3) + 2*m, m = 0..7, as its
// bytes m.  So if input lanes 2m and 2m+1 address columns c..c+7 and
// c+8..c+15 of weight row k0 + m, output lane t holds rows k0..k0+7 of column
// c + t: 8 consecutive k of one n.  Read j (0..3) of lane group g takes
// k0 = 32*g + 8*j, giving the lane bytes 8j..8j+7 of the MFMA fragment with
// k = 32*g .. 32*g+31 -- the A fragments' k <-> (lane, byte) mapping.  The
// fragment's 16 rows are the 16 consecutive columns 16*tn .. 16*tn+15 of the
// wave's 64.  Returns the lane's LDS byte offset for read j of tile tn
// (wn = the wave's column quarter).
__device__ __forceinline__ int frag_off_w(int lane, int wn, int tn, int j)
{
    const int g = lane >> 4;
    const int m = (lane & 15) >> 1;
    const int p = lane & 1;
    const int r = 32 * g + 8 * j + m;
    return r * 256 + (((4 * wn + tn) ^ swz_w(r)) << 4) + 8 * p;
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

__device__ __forceinline__ v8i load_frag_w(const uint8_t* base, int off0, int off1, int off2,
                                           int off3)
{
    const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + off0));
    const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + off1));
    const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + off2));
    const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + off3));
    v8i f;
    f[0] = r0[0]; f[1] = r0[1]; f[2] = r1[0]; f[3] = r1[1];
    f[4] = r2[0]; f[5] = r2[1]; f[6] = r3[0]; f[7] = r3[1];
    return f;
}

// `base` is an LDS array and `off` the slice's byte offset in it; each read
// is a single offset from the array so the compiler keeps track of which LDS
// object it touches (and does not wait for copies into the other stage).
__device__ __forceinline__ v8i load_frag(const uint8_t* base, int off, FragOff fo)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(&base[off + fo.lo]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&base[off + fo.hi]);
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

// BF16 operand fragment (v_mfma_f32_16x16x32_bf16): lane l holds 8 values of
// row (l & 15), i.e. one 16-byte chunk.  A 128-byte K-block is two MFMA
// K-steps: chunk (l >> 4) in the first and 4 + (l >> 4) in the second, with
// the same lane mapping for A and B.  `lo` / `hi` are the two chunk offsets.
__device__ __forceinline__ FragOff frag_off_bf16(int r, int lane, int mask)
{
    const int c0 = lane >> 4;
    return {r * BK + ((c0 ^ mask) << 4), r * BK + (((c0 + 4) ^ mask) << 4)};
}

__device__ __forceinline__ v8bf load_chunk_bf16(const uint8_t* base, int off)
{
    const uint4 v = *reinterpret_cast<const uint4*>(&base[off]);
    return __builtin_bit_cast(v8bf, v);
}

// One 16x16x128 E4M3 x E4M3 product with a zero accumulator input.  The
// builtin is the scaled form; with its scale operands the compile-time
// constant 0 the compiler emits the unscaled v_mfma_f32_16x16x128_f8f6f4,
// i.e. unit scales.  (The scaled instruction reads E8M0 bytes: 127 is 1.0,
// and a byte of 0 at run time would scale the product by 2^-127 -- pinned,
// with the emitted form's unit scale, by tests/test_gpu_mfma_accum.py.)
__device__ __forceinline__ v4f mfma_e4m3(const v8i& x, const v8i& y)
{
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// One K-block (128 deep) staged in LDS: A and B code slices and their scales.
struct Stage {
    uint8_t a[TILE_BYTES];
    uint8_t b[TILE_BYTES];
    float sa[BM];        // sA of the tile's 256 rows
    float sb[BN];        // WGRAD: sB of the tile's 256 columns; else [0], [1]
};

// A wave-uniform pointer held in scalar registers.  Going through
// readfirstlane keeps the compiler from folding per-lane offsets into the
// base (which would hoist 64-bit per-lane addresses out of the K loop); the
// loads then use the scalar-base + 32-bit vector-offset form.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Staging of one K-block: every wave copies 32 rows of A and 32 rows of B
// (4 + 4 LDS-DMA instructions of 1 KB, 16 bytes per lane).  Lane L of
// instruction i fills LDS row 32*wave + 8*i + L/8 at chunk position L%8, so it
// fetches the logical chunk the swizzle stores there; rows past the end of
// the matrix read the tile's last row instead (their results are never
// stored).  `At` / `Bt` point at the tile's first row; the 64-bit row base
// and K-block offset stay in scalar registers and each lane adds a 32-bit
// offset (row < 256 and K <= 2^24 keep it below 2^32).
// Wave 0 also copies the 256 sA values, wave 1 the sB values.
template <int MODE>
__device__ __forceinline__ void issue_stage(Stage& st, const uint8_t* At, const float* SA,
                                            const uint8_t* Bt, const float* SB, int kb, int m0,
                                            int n0, int rows_a, int rows_b, int M, int N, int K,
                                            int KB, int wave, int lane)
{
    const uint8_t* ab = uniform_ptr(At + (size_t)kb * BK);
    const int r0 = 32 * wave + (lane >> 3);
    if constexpr (b_kn(MODE)) {
        // B = rows kb*128 .. +127 of the [K][N] codes, columns n0 .. n0+255
        // (N-contiguous, N = the row pitch); each wave copies 16 rows, lane L of instruction i
        // fills row 16*wave + 4*i + L/16 at unit position L % 16.  Columns past N
        // (a half tile) read the row's last 16 bytes instead (never stored).
        const uint8_t* wb = uniform_ptr(Bt + (size_t)kb * BK * (size_t)N);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * wave + 4 * i + (lane >> 4);
            const int col = min(n0 + 16 * ((lane & 15) ^ swz_w(row)), N - 16);
            const uint8_t* rb = uniform_ptr(wb + (size_t)(16 * wave + 4 * i) * (size_t)N);
            const uint32_t bo = (uint32_t)(lane >> 4) * (uint32_t)N + (uint32_t)col;
            __builtin_amdgcn_global_load_lds(rb + bo, (lds_void*)(st.b + (16 * wave + 4 * i) * 256), 16, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + 8 * i;
        const uint32_t ca = 16u * (uint32_t)((lane & 7) ^ swz(row));
        const uint32_t ao = (uint32_t)min(row, rows_a - 1) * (uint32_t)K + ca;
        __builtin_amdgcn_global_load_lds(ab + ao, (lds_void*)(st.a + (32 * wave + 8 * i) * BK), 16, 0, 0);
        if constexpr (!b_kn(MODE)) {
            const uint8_t* bb = uniform_ptr(Bt + (size_t)kb * BK);
            const uint32_t cb = 16u * (uint32_t)((lane & 7) ^ swz_stage_b<MODE>(row));
            const uint32_t bo = (uint32_t)min(row, rows_b - 1) * (uint32_t)K + cb;
            __builtin_amdgcn_global_load_lds(bb + bo, (lds_void*)(st.b + (32 * wave + 8 * i) * BK), 16, 0, 0);
        }
    }
    if constexpr (MODE == MODE_BF16)
        return;                                  // no block scales
    if (wave == 0) {
        const float* sab = uniform_ptr(SA + (size_t)kb * M);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(sab + min(m0 + 64 * j + lane, M - 1),
                                             (lds_void*)(st.sa + 64 * j), 4, 0, 0);
    } else if (wave == 1) {
        if constexpr (MODE == MODE_WGRAD) {
            __builtin_amdgcn_global_load_lds(uniform_ptr(SB + (size_t)kb * N) + min(n0 + 4 * lane, N - 4),
                                             (lds_void*)(st.sb), 16, 0, 0);
        } else if (lane < 2) {
            const int nb = min(n0 / BK + lane, N / BK - 1);
            const size_t idx = (MODE == MODE_FWD || MODE == MODE_FWD_T) ? (size_t)nb * KB + kb
                                                                        : (size_t)kb * (N / BK) + nb;
            __builtin_amdgcn_global_load_lds(SB + idx, (lds_void*)(st.sb), 4, 0, 0);
        }
    }
}

template <int MODE, int OUT>
__global__ __launch_bounds__(NTHREADS) void gemm_bs_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA,
    const uint8_t* __restrict__ B, const float* __restrict__ SB,
    void* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n, int splits,
    int kb_per_split)
{
    __shared__ __attribute__((aligned(16))) Stage stage0;
    __shared__ __attribute__((aligned(16))) Stage stage1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2;        // 0..1
    const int wn = wave & 3;         // 0..3

    // ---- work units: (split, output tile), XCD-compact and grouped along M.
    // The grid is persistent: work-group g takes units g, g + G, g + 2G, ...
    // (G = gridDim.x, a multiple of 8 whenever it is below the unit count).
    // Work-groups are dealt to the 8 XCDs round-robin, so unit u runs on XCD
    // u % 8; the remap below gives each XCD a contiguous range of units, so
    // the tiles that run together on one XCD share A and B panels in its L2.
    const int total = tiles_m * tiles_n * splits;
    const int tiles = tiles_m * tiles_n;
    const int KB = K / BK;
    struct Unit {
        int m0, n0, split, kb_begin, kb_end;
    };
    auto unit_of = [&](int u) __attribute__((always_inline)) -> Unit {
        int w = u;
        if ((total & 7) == 0)
            w = (w & 7) * (total >> 3) + (w >> 3);
        const int split = w / tiles;
        const int tile = w - split * tiles;
        const int group_size = GROUP_M * tiles_n;
        const int group = tile / group_size;
        const int first_m = group * GROUP_M;
        const int gm = min(tiles_m - first_m, GROUP_M);
        const int in_group = tile - group * group_size;
        const int tile_m = first_m + in_group % gm;
        const int tile_n = in_group / gm;
        const int kb_begin = split * kb_per_split;
        return {tile_m * BM, tile_n * BN, split, kb_begin, min(KB, kb_begin + kb_per_split)};
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int sm = 0; sm < TM; ++sm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
            acc[sm][tn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // One K-block from a staged buffer: 32 MFMAs in 8 rows of 4 (one row =
    // one 16-row A fragment against the wave's 4 B fragments).  The partial
    // of MFMA tile (sm, tn) is folded into its accumulator (one FMA per
    // element with the block scale) in the next row, just before MFMA
    // (sm+1, tn) overwrites it: four MFMAs after it was issued, so the fold
    // never waits for the matrix core and the partials need a single set of
    // registers.  The A fragment of row sm+1 is read from LDS while row sm is
    // multiplied.
    //
    // FWD / DGRAD issue the MFMA with the B-side fragment first: a lane's 4
    // accumulator rows are 4 consecutive n of one m, sA is one value per lane
    // and tile, sB one value per wave.  The last row's partials are carried
    // into the next K-block and folded during its first row (with the scale
    // of the block they belong to), so no K-block ends on a chain of FMAs
    // waiting for its last MFMAs.  The carried partials start at zero with a
    // zero scale, and the first fold adds +0 to +0.
    //
    // WGRAD (per-column sB) issues it with the A-side fragment first: a
    // lane's 4 rows are 4 consecutive m of one n, so it holds 4 sB values per
    // K-block and one float4 of sA per tile.
    const FragOff fo = frag_off(lane);
    const FragOff fob = (MODE == MODE_WGRAD) ? fo : frag_off_b(lane);
    // [K][N] modes: per tile, the lane's offset of transpose read j = 0 (read
    // j adds 8 weight rows, 2048 bytes)
    int fow[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
        fow[tn] = frag_off_w(lane, wn, tn, 0);
    const int a_off = wm * WM * BK;    // this wave's 128 A rows
    const int b_off = wn * WN * BK;    // this wave's 64 B rows
    v4f p[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
        p[tn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float sc_carry = 0.0f;
    auto fold_row = [&](int sm, float sc) __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[sm][tn][r] = __builtin_fmaf(p[tn][r], sc, acc[sm][tn][r]);
    };
    // `after_row0` (the next stage's LDS copy) runs once row 0's MFMAs are
    // issued: with no copy outstanding the compiler can wait for each of the
    // block's first fragments individually (while an LDS-DMA copy is in
    // flight it makes every LDS-read wait a full lgkmcnt(0)).
    auto compute = [&](const Stage& st, auto&& after_row0) __attribute__((always_inline)) {
        if constexpr (MODE == MODE_BF16) {
            // B-first like FWD (the same store-friendly B row order); the
            // MFMAs accumulate into acc directly.  Within a row the four tiles
            // take K-step 0, then K-step 1, so dependent accumulations are
            // four MFMAs apart.
            const int ra = lane & 15;
            const int rb = 8 * ((lane & 15) >> 2) + (lane & 3);
            const FragOff fa = frag_off_bf16(ra, lane, swz(ra));
            const FragOff fb = frag_off_bf16(rb, lane, swz_b(rb));
            v8bf bf[TN][2];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                __builtin_amdgcn_sched_barrier(0);
                bf[tn][0] = load_chunk_bf16(st.b, b_off + b_tile_rows(tn) * BK + fb.lo);
                bf[tn][1] = load_chunk_bf16(st.b, b_off + b_tile_rows(tn) * BK + fb.hi);
            }
            v8bf af0 = load_chunk_bf16(st.a, a_off + fa.lo);
            v8bf af1 = load_chunk_bf16(st.a, a_off + fa.hi);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sm = 0; sm < TM; ++sm) {
                __builtin_amdgcn_sched_barrier(0);
                v8bf an0, an1;
                if (sm + 1 < TM) {
                    an0 = load_chunk_bf16(st.a, a_off + 16 * (sm + 1) * BK + fa.lo);
                    an1 = load_chunk_bf16(st.a, a_off + 16 * (sm + 1) * BK + fa.hi);
                }
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    acc[sm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[tn][0], af0, acc[sm][tn], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    acc[sm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[tn][1], af1, acc[sm][tn], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (sm + 1 < TM) {
                    af0 = an0;
                    af1 = an1;
                }
                if (sm == 0) {
                    after_row0();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (MODE == MODE_WGRAD) {
            v8i bf[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                bf[tn] = load_frag(st.b, b_off + 16 * tn * BK, fo);
            float sbn[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                sbn[tn] = st.sb[wn * WN + 16 * tn + (lane & 15)];
            v4f sa_prev = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sm = 0; sm < TM; ++sm) {
                const v8i af = load_frag(st.a, a_off + 16 * sm * BK, fo);
                const v4f sa4 = *reinterpret_cast<const v4f*>(&st.sa[wm * WM + 16 * sm + 4 * (lane >> 4)]);
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    if (sm > 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[sm - 1][tn][r] = __builtin_fmaf(p[tn][r], sa_prev[r] * sbn[tn], acc[sm - 1][tn][r]);
                    }
                    p[tn] = mfma_e4m3(af, bf[tn]);
                }
                sa_prev = sa4;
                if (sm == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    after_row0();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[TM - 1][tn][r] = __builtin_fmaf(p[tn][r], sa_prev[r] * sbn[tn], acc[TM - 1][tn][r]);
        } else {
            // Row 0's A fragment, then B[0..3] in MFMA order, each group fenced:
            // LDS reads complete in issue order, so MFMA (0, tn) waits only
            // for A and B[0..tn], not for every read of the block's head.
            v8i af = load_frag(st.a, a_off, fo);
            v8i bf[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (b_kn(MODE))
                    bf[tn] = load_frag_w(st.b, fow[tn], fow[tn] + 2048, fow[tn] + 4096,
                                         fow[tn] + 6144);
                else
                    bf[tn] = load_frag(st.b, b_off + b_tile_rows(tn) * BK, fob);
            }
            __builtin_amdgcn_sched_barrier(0);
            const float sb_wave = st.sb[(wn * WN) / BK];
            float sa = st.sa[wm * WM + (lane & 15)];
#pragma unroll
            for (int sm = 0; sm < TM; ++sm) {
                __builtin_amdgcn_sched_barrier(0);
                v8i af_next;
                float sa_next = 0.0f;
                if (sm + 1 < TM) {
                    af_next = load_frag(st.a, a_off + 16 * (sm + 1) * BK, fo);
                    sa_next = st.sa[wm * WM + 16 * (sm + 1) + (lane & 15)];
                }
                // fold row sm-1 (row TM-1 of the previous K-block when sm == 0)
                const float sc_prev = sc_carry;
                const int fold_sm = (sm == 0) ? TM - 1 : sm - 1;
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[fold_sm][tn][r] = __builtin_fmaf(p[tn][r], sc_prev, acc[fold_sm][tn][r]);
                    p[tn] = mfma_e4m3(bf[tn], af);
                    __builtin_amdgcn_sched_barrier(0);   // MFMAs in tn order
                }
                sc_carry = sa * sb_wave;
                if (sm + 1 < TM) {
                    af = af_next;
                    sa = sa_next;
                }
                if (sm == 0) {
                    after_row0();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- epilogue of one unit: C (+)= acc ------------------------------------
    // OUT_PARTIAL writes the unit's split-K partial to plane `split` of C.
    auto store4 = [&](size_t idx, int split, v4f v) __attribute__((always_inline)) {   // 4 consecutive FP32
        if constexpr (OUT == OUT_FP32) {
            *reinterpret_cast<v4f*>(static_cast<float*>(C) + idx) = v;
        } else if constexpr (OUT == OUT_FP32_ACC) {
            v4f* dst = reinterpret_cast<v4f*>(static_cast<float*>(C) + idx);
            *dst = *dst + v;
        } else if constexpr (OUT == OUT_PARTIAL) {
            *reinterpret_cast<v4f*>(static_cast<float*>(C) + (size_t)split * M * N + idx) = v;
        }
    };
    auto store1 = [&](size_t idx, int split, float v) __attribute__((always_inline)) {        // one element
        if constexpr (OUT == OUT_BF16) {
            static_cast<uint16_t*>(C)[idx] = (uint16_t)pack_bf16(v, 0.0f);
        } else if constexpr (OUT == OUT_FP32) {
            static_cast<float*>(C)[idx] = v;
        } else if constexpr (OUT == OUT_FP32_ACC) {
            float* dst = static_cast<float*>(C) + idx;
            *dst = *dst + v;
        } else {
            static_cast<float*>(C)[(size_t)split * M * N + idx] = v;
        }
    };
    auto epilogue = [&](const Unit& t) __attribute__((always_inline)) {
        if constexpr (MODE != MODE_WGRAD && MODE != MODE_BF16)
            fold_row(TM - 1, sc_carry);               // the unit's last row
        if ((t.n0 + wn * WN) >= N)
            return;
        if constexpr (MODE == MODE_WGRAD) {
            // lane: column n = n_lane + 16*tn, rows m = m_lane + 16*sm + r
            const int n_lane = t.n0 + wn * WN + (lane & 15);
            const int m_lane = t.m0 + wm * WM + 4 * (lane >> 4);
#pragma unroll
            for (int sm = 0; sm < TM; ++sm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m_lane + 16 * sm + r;
                    if (m < M) {
#pragma unroll
                        for (int tn = 0; tn < TN; ++tn)
                            store1((size_t)m * N + n_lane + 16 * tn, t.split, acc[sm][tn][r]);
                    }
                }
        } else if constexpr (b_kn(MODE)) {
            // lane: row m = m_lane + 16*sm; columns n_lane + 16*tn + r (the
            // fragments' natural column order, g = lane >> 4).  FP32: one
            // 16-byte store per tile.  bf16: lane groups g and g ^ 1 (lanes l
            // and l ^ 16, the same row) trade halves of tiles 2q and 2q + 1,
            // so an even group holds columns 16*(2q) + 4g .. +7 and an odd one
            // 16*(2q+1) + 4g - 4 .. +7; across the four groups that is 64
            // contiguous bytes of the row per tile pair, one 16-byte store per
            // lane, as in the other modes.
            const int g = lane >> 4;
            const bool odd = (g & 1) != 0;
            const int m_lane = t.m0 + wm * WM + (lane & 15);
            const int n_lane = t.n0 + wn * WN + 4 * g;
#pragma unroll
            for (int sm = 0; sm < TM; ++sm) {
                const int m = m_lane + 16 * sm;
                if (m >= M)
                    continue;                  // lanes l and l ^ 16 share m
                const size_t idx = (size_t)m * N + n_lane;
                if constexpr (OUT == OUT_BF16) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int ta = 2 * q, tb = 2 * q + 1;
                        const uint32_t a0 = pack_bf16(acc[sm][ta][0], acc[sm][ta][1]);
                        const uint32_t a1 = pack_bf16(acc[sm][ta][2], acc[sm][ta][3]);
                        const uint32_t b0 = pack_bf16(acc[sm][tb][0], acc[sm][tb][1]);
                        const uint32_t b1 = pack_bf16(acc[sm][tb][2], acc[sm][tb][3]);
                        // swizzle pattern: lane ^ 16 within each half wave
                        const uint32_t y0 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(odd ? a0 : b0), 0x401F);
                        const uint32_t y1 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(odd ? a1 : b1), 0x401F);
                        const v4u w = odd ? v4u{y0, y1, b0, b1} : v4u{a0, a1, y0, y1};
                        const size_t col = odd ? idx + 16 * tb - 4 : idx + 16 * ta;
                        // Ordinary stores: measured on the MI355X, non-temporal
                        // ones made this layout's L2 write 1.4x the output's
                        // bytes back to memory and ran 2-3% slower; these write
                        // 1.015x.
                        *reinterpret_cast<v4u*>(static_cast<uint16_t*>(C) + col) = w;
                    }
                } else {
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        store4(idx + 16 * tn, t.split, acc[sm][tn]);
                }
            }
        } else {
            // lane: row m = m_lane + 16*sm; columns n_lane + b_tile_rows(tn) + r,
            // i.e. 8 consecutive columns from tiles 0, 1 and 8 more, 32 columns
            // on, from tiles 2, 3 (the B fragments' row order, frag_off_b)
            const int m_lane = t.m0 + wm * WM + (lane & 15);
            const int n_lane = t.n0 + wn * WN + 8 * (lane >> 4);
#pragma unroll
            for (int sm = 0; sm < TM; ++sm) {
                const int m = m_lane + 16 * sm;
                if (m >= M)
                    continue;
                const size_t idx = (size_t)m * N + n_lane;
                if constexpr (OUT == OUT_BF16) {
                    uint32_t w[8];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) {
                        w[2 * tn] = pack_bf16(acc[sm][tn][0], acc[sm][tn][1]);
                        w[2 * tn + 1] = pack_bf16(acc[sm][tn][2], acc[sm][tn][3]);
                    }
                    // Non-temporal: the output is not read again by this
                    // kernel.  Measured on the MI355X against ordinary stores:
                    // 2% faster on a 16384 x 16384 output, equal on narrower
                    // ones, at a cost of 7-18% more bytes written back.
                    v4u* dst = reinterpret_cast<v4u*>(static_cast<uint16_t*>(C) + idx);
                    __builtin_nontemporal_store(v4u{w[0], w[1], w[2], w[3]}, dst);
                    __builtin_nontemporal_store(v4u{w[4], w[5], w[6], w[7]}, dst + 4);
                } else {
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        store4(idx + b_tile_rows(tn), t.split, acc[sm][tn]);
                }
            }
        }
    };
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int sm = 0; sm < TM; ++sm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                acc[sm][tn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
            p[tn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        sc_carry = 0.0f;
    };

    // ---- main loop over the steps (unit, K-block) of this work-group -------
    // Two statically named LDS stages alternate, one barrier per step.  At
    // the top of a step the wait covers this wave's share of the stage and
    // the barrier the other waves' (a plain s_barrier: every LDS read of the
    // previous stage was consumed by an MFMA before it).  Then
    //   * the previous unit's epilogue runs if it is due, so its stores drain
    //     while this block is multiplied, and the accumulators restart;
    //   * the LDS copy of the next step's block -- the next K-block, or the
    //     first one of the next unit -- is issued into the other stage;
    //   * the block is multiplied.
    // A work-group therefore never idles between units: the next unit's
    // first block is already in LDS when the last block of a unit is done.
    auto issue = [&](Stage& st, const Unit& t, int kb) __attribute__((always_inline)) {
        const uint8_t* At = A + (size_t)t.m0 * K;
        const uint8_t* Bt = b_kn(MODE) ? B : B + (size_t)t.n0 * K;
        issue_stage<MODE>(st, At, SA, Bt, SB, kb, t.m0, t.n0, min(M - t.m0, BM),
                          min(N - t.n0, BN), M, N, K, KB, wave, lane);
    };
    const int G = gridDim.x;
    int u = blockIdx.x;
    Unit cur = unit_of(u);
    int kb = cur.kb_begin;
    bool have_next = u + G < total;
    Unit nxt = unit_of(have_next ? u + G : u);
    Unit done = cur;
    bool pending = false;
    issue(stage0, cur, kb);
    auto step = [&](Stage& st, Stage& other) __attribute__((always_inline)) -> bool {
        // vmcnt(0): this wave's share of the stage has landed.  lgkmcnt(0)
        // costs nothing here (every LDS read of the previous step was
        // consumed by an MFMA) but clears the compiler's view of the last
        // copy as a pending LDS event, which would otherwise turn the block
        // head's per-fragment waits into full ones.  The hardware tracks
        // LDS-DMA copies with vmcnt only (checked on the device: LDS still
        // holds the old data after lgkmcnt(0), the new data after vmcnt(0)).
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (pending) {
            epilogue(done);
            reset();
            pending = false;
        }
        const bool unit_ends = kb + 1 >= cur.kb_end;
        auto copy_next = [&]() __attribute__((always_inline)) {
            if (!unit_ends)
                issue(other, cur, kb + 1);
            else if (have_next)
                issue(other, nxt, nxt.kb_begin);
        };
        // Waves whose columns lie beyond N only copy.  Their copy comes after
        // the compute region: an LDS copy on any path into the block head
        // would make the compiler wait for all of the head's reads at once.
        const bool active = (cur.n0 + wn * WN) < N;
        if (active)
            compute(st, copy_next);
        __builtin_amdgcn_sched_barrier(0);
        if (!active)
            copy_next();
        if (!unit_ends) {
            ++kb;
            return true;
        }
        done = cur;
        pending = true;
        if (!have_next)
            return false;
        u += G;
        cur = nxt;
        kb = cur.kb_begin;
        have_next = u + G < total;
        nxt = unit_of(have_next ? u + G : u);
        return true;
    };
    while (step(stage0, stage1) && step(stage1, stage0)) {
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
    epilogue(done);
}

// Sum of the split-K partials in split order, then the requested output.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            void* __restrict__ C, int64_t count4,
                                                            int splits, int64_t plane)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count4; i += stride) {
        v4f s = *reinterpret_cast<const v4f*>(ws + 4 * i);
        for (int z = 1; z < splits; ++z)
            s = s + *reinterpret_cast<const v4f*>(ws + (size_t)z * plane + 4 * i);
        if constexpr (OUT == OUT_BF16) {
            uint2 o;
            o.x = pack_bf16(s[0], s[1]);
            o.y = pack_bf16(s[2], s[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + 4 * i) = o;
        } else if constexpr (OUT == OUT_FP32) {
            *reinterpret_cast<v4f*>(static_cast<float*>(C) + 4 * i) = s;
        } else {
            v4f* dst = reinterpret_cast<v4f*>(static_cast<float*>(C) + 4 * i);
            *dst = *dst + s;
        }
    }
}

// Diagnostic: one matrix-core instruction of the given form on raw per-lane
// operand bytes, with a zero accumulator input.  a, b: u8 [64][32] (lane l's
// operand bytes at 32*l; the 8-byte forms use the first 8, the bf16 form the
// first 16); d: f32 [64][16] (lane l's result registers at 16*l, unused
// slots zero).  One wave.  Lets a test see how each form adds its products.
//   form 0: v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3), as the GEMM issues it
//   form 1: v_mfma_f32_32x32x64_f8f6f4  (E4M3 x E4M3)
//   form 2: v_mfma_f32_16x16x32_fp8_fp8
//   form 3: v_mfma_f32_32x32x16_fp8_fp8
//   form 4: v_mfma_f32_16x16x32_bf16
//   form 5: v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0 scale bytes
//           scale_a, scale_b taken from the arguments at run time (opsel 0)
typedef float v16f __attribute__((ext_vector_type(16)));
typedef long v1l;
__global__ __launch_bounds__(64) void probe_mfma_kernel(int form, const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ b, int scale_a,
                                                        int scale_b, float* __restrict__ d)
{
    const int lane = threadIdx.x;
    const v8i av = *reinterpret_cast<const v8i*>(a + 32 * lane);
    const v8i bv = *reinterpret_cast<const v8i*>(b + 32 * lane);
    float out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        out[i] = 0.0f;
    const v4f z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (form == 0 || form == 2 || form == 4 || form == 5) {
        v4f r = z4;
        if (form == 0) {
            r = mfma_e4m3(av, bv);
        } else if (form == 2) {
            const long al = (long)(uint32_t)av[0] | ((long)(uint32_t)av[1] << 32);
            const long bl = (long)(uint32_t)bv[0] | ((long)(uint32_t)bv[1] << 32);
            r = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(al, bl, z4, 0, 0, 0);
        } else if (form == 4) {
            v8bf ab, bb;
            const uint4 au = {(uint32_t)av[0], (uint32_t)av[1], (uint32_t)av[2], (uint32_t)av[3]};
            const uint4 bu = {(uint32_t)bv[0], (uint32_t)bv[1], (uint32_t)bv[2], (uint32_t)bv[3]};
            ab = __builtin_bit_cast(v8bf, au);
            bb = __builtin_bit_cast(v8bf, bu);
            r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, z4, 0, 0, 0);
        } else {
            r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z4, 0, 0, 0, scale_a, 0,
                                                                scale_b);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = r[i];
    } else {
        const v16f z16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                          0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        v16f r = z16;
        if (form == 1) {
            r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, z16, 0, 0, 0, 0, 0, 0);
        } else {
            const long al = (long)(uint32_t)av[0] | ((long)(uint32_t)av[1] << 32);
            const long bl = (long)(uint32_t)bv[0] | ((long)(uint32_t)bv[1] << 32);
            r = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(al, bl, z16, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            out[i] = r[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        d[16 * lane + i] = out[i];
}

hipError_t launch_probe_mfma(int form, const uint8_t* a, const uint8_t* b, int scale_a,
                             int scale_b, float* d, hipStream_t stream)
{
    return launch_kernel(probe_mfma_kernel, dim3(1), dim3(64), stream, form, a, b, scale_a,
                         scale_b, d);
}

// Split-K factor: only when the tile grid leaves most of the 256 CUs idle.
// Picks the smallest split that best fills whole waves of 256 workgroups
// while keeping at least 8 K-blocks per split.
static int choose_splits(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t KB = K / BK;
    if (tiles >= 256 || KB < 16)
        return 1;
    int best = 1;
    double best_eff = 0.0;
    for (int s = 1; s <= 8; ++s) {
        if (KB / s < 8)
            break;
        const int64_t units = tiles * s;
        const int64_t waves = (units + 255) / 256;
        const double eff = (double)units / (double)(waves * 256);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = s;
        }
    }
    return best;
}

size_t gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K)
{
    (void)mode;
    const int s = choose_splits(M, N, K);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Persistent grid: one work-group per compute unit of the stream's device
// (the kernel holds one work-group per CU), a multiple of 8 so the units of
// one XCD stay contiguous; fewer when there are fewer units.
static int persistent_grid(int units, hipStream_t stream)
{
    int dev = 0;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess)
            dev = 0;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (units <= cus)
        return units;
    return cus >= 8 ? cus / 8 * 8 : cus;
}

template <int MODE>
static hipError_t launch_mode(int out, const uint8_t* a, const float* sa, const uint8_t* b,
                              const float* sb, void* c, void* ws, int M, int N, int K,
                              int splits, hipStream_t stream)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int KB = K / BK;
    const int kbps = (KB + splits - 1) / splits;
    if (KB <= 0 || (splits - 1) * kbps >= KB)   // every unit needs a K-block
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)persistent_grid(tiles_m * tiles_n * splits, stream));
    const dim3 block(NTHREADS);
    if (splits > 1) {
        const hipError_t e = launch_kernel(gemm_bs_kernel<MODE, OUT_PARTIAL>, grid, block, stream,
                                           a, sa, b, sb, ws, M, N, K, tiles_m, tiles_n, splits, kbps);
        if (e != hipSuccess)
            return e;
        const int64_t count4 = (int64_t)M * N / 4;
        const int64_t blocks = (count4 + 255) / 256;
        const dim3 rgrid((unsigned)(blocks < 8192 ? blocks : 8192));
        const float* wsf = static_cast<const float*>(ws);
        const int64_t total = (int64_t)M * N;
        if (out == OUT_BF16)
            return launch_kernel(splitk_reduce_kernel<OUT_BF16>, rgrid, dim3(256), stream, wsf, c,
                                 count4, splits, total);
        if (out == OUT_FP32)
            return launch_kernel(splitk_reduce_kernel<OUT_FP32>, rgrid, dim3(256), stream, wsf, c,
                                 count4, splits, total);
        return launch_kernel(splitk_reduce_kernel<OUT_FP32_ACC>, rgrid, dim3(256), stream, wsf, c,
                             count4, splits, total);
    }
    if (out == OUT_BF16)
        return launch_kernel(gemm_bs_kernel<MODE, OUT_BF16>, grid, block, stream, a, sa, b, sb, c,
                             M, N, K, tiles_m, tiles_n, 1, KB);
    if (out == OUT_FP32)
        return launch_kernel(gemm_bs_kernel<MODE, OUT_FP32>, grid, block, stream, a, sa, b, sb, c,
                             M, N, K, tiles_m, tiles_n, 1, KB);
    return launch_kernel(gemm_bs_kernel<MODE, OUT_FP32_ACC>, grid, block, stream, a, sa, b, sb, c,
                         M, N, K, tiles_m, tiles_n, 1, KB);
}

size_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const int s = choose_splits(M, N, 2 * K);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                               void* c, void* ws, hipStream_t stream)
{
    const int64_t kbytes = 2 * K;
    const int splits = choose_splits(M, N, kbytes);
    return launch_mode<MODE_BF16>(OUT_BF16, static_cast<const uint8_t*>(a), nullptr,
                                  static_cast<const uint8_t*>(b), nullptr, c, ws, (int)M, (int)N,
                                  (int)kbytes, splits, stream);
}

hipError_t launch_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                       const float* sa, const uint8_t* b, const float* sb, void* c, int out_fp32,
                       int accumulate, void* ws, hipStream_t stream)
{
    const int out = out_fp32 ? (accumulate ? OUT_FP32_ACC : OUT_FP32) : OUT_BF16;
    const int splits = choose_splits(M, N, K);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (mode) {
    case MODE_FWD:   return launch_mode<MODE_FWD>(out, a, sa, b, sb, c, ws, m, n, k, splits, stream);
    case MODE_DGRAD: return launch_mode<MODE_DGRAD>(out, a, sa, b, sb, c, ws, m, n, k, splits, stream);
    case 3:          // the C ABI's PURO_GEMM_DGRAD_W
        return launch_mode<MODE_DGRAD_W>(out, a, sa, b, sb, c, ws, m, n, k, splits, stream);
    case 4:          // the C ABI's PURO_GEMM_FWD_T
        return launch_mode<MODE_FWD_T>(out, a, sa, b, sb, c, ws, m, n, k, splits, stream);
    default:         return launch_mode<MODE_WGRAD>(out, a, sa, b, sb, c, ws, m, n, k, splits, stream);
    }
}

// ---- the allocation-free variant: split-K partials in a static device array --
// Callers that cannot allocate (code under graph capture, tight serving
// loops) get the split-K workspace from `scratch`, a fixed array that every
// GPU the library runs on holds until the process ends.  In host code the
// array's name is only a stand-in: its device address, which differs per
// GPU, comes from hipGetSymbolAddress, looked up once per device with that
// device current, and only that address is passed to the kernels.  Every
// call on one GPU shares the array; each split overwrites its whole plane of
// partials before the reduce reads it, so nothing needs clearing, and calls
// that overlap on one GPU (other streams, other threads) race.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `dev` (looked up on first use).
hipError_t scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess)
            return e;
        if (prev != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (prev != dev) {
            const hipError_t r = hipSetDevice(prev);
            if (e == hipSuccess)
                e = r;
        }
        if (e != hipSuccess)
            return e;
        if (!ptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

size_t gemm_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                               const float* sa, const uint8_t* b, const float* sb, void* c,
                               int out_fp32, int accumulate, hipStream_t stream)
{
    void* ws = nullptr;
    if (gemm_workspace_bytes(mode, M, N, K) > 0) {
        int dev = 0;
        hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if ((e = scratch_address(dev, &ws)) != hipSuccess)
            return e;
    }
    return launch_gemm(mode, M, N, K, a, sa, b, sb, c, out_fp32, accumulate, ws, stream);
}

}  // namespace puro
