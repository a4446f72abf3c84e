// Device-side building blocks shared by the forward and backward kernels
// (gfx950 / CDNA4 only).
//
// MFMA operand layout used throughout (32x32 output tiles, wave64):
//   A (M x K) and B (K x N) fragments: lane l supplies row (A) / column (B)
//   l % 32 and the E contraction elements [E*(l/32), E*(l/32)+E) of the step.
//   C/D (32 x 32 fp32, 16 registers): lane l holds column l % 32 and rows
//   8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// Only the C/D layout has to be right for correctness: the contraction index
// of A and B may be permuted freely as long as both sides use the same
// permutation, which the kernels exploit to feed accumulators straight back
// into the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-element-type MFMA traits.
//   E  : contraction elements one lane supplies per MFMA
//   KS : contraction length of one MFMA (= 2 E)
//   CH : elements in a 16-byte chunk (unit of global loads)
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int E = 8, KS = 16, CH = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int E = 1, KS = 2, CH = 4;
    typedef float frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// 16-byte chunk of T.
template <typename T> struct Chunk { u32x4 v; };

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zeros (hardware range check), which is how rows past N read as 0.
// Word 3 = 0x00020000: 32-bit data format, as untyped buffer loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ---- LDS tiles written by direct-to-LDS loads (no padding possible) ----
// Rows of RB = 256 bytes (16 slots of 16 B) or 128 bytes (8 slots).  Logical
// 16-byte chunk c of row r lives in slot swz(r, c).  Measured on gfx950 (64 banks;
// 16 lanes per cycle for 16-byte reads, 32 lanes for the 8-byte transpose reads),
// the layouts below make both access patterns conflict-free:
//   (a) 16 lanes reading the same chunk of 16 consecutive rows (row fragments);
//   (b) 32 lanes reading 4 consecutive rows x 4 adjacent chunks (transpose reads).
// 256-byte rows: slot = pi(c) ^ f(r), where pi sends chunk bit 1 to slot bit 3 (so
// the two 16-lane halves of (b) use opposite bank halves) and f is a permutation
// of the row's low four bits.  128-byte rows: slot = c ^ g(r / 2), g flips slot
// bit 2 between even and odd row pairs.
__device__ __forceinline__ int swz_pi(int c)
{
    return (c & 1) | (((c >> 1) & 1) << 3) | (((c >> 2) & 1) << 1) | (((c >> 3) & 1) << 2);
}
__device__ __forceinline__ int swz_pi_inv(int s)
{
    return (s & 1) | (((s >> 3) & 1) << 1) | (((s >> 1) & 1) << 2) | (((s >> 2) & 1) << 3);
}
__device__ __forceinline__ int swz_f(int r)
{
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (r & 8);
}
__device__ __forceinline__ int swz_g(int r)
{
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | ((x >> 1) & 3);
}
//
// A second, XOR-only layout (FAST = false) is conflict-free for (a) and for each
// 16-lane half of (b) but not for (b) as a whole.  Its offsets for the four
// 32-column tiles and for the second transpose read are constant distances from
// two per-lane values, which saves registers and address arithmetic; the kernel
// that runs one wave per SIMD (nothing to hide extra VALU work) uses it.
__device__ __forceinline__ int swz_x256(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
__device__ __forceinline__ int swz_x128(int r)
{
    const int x = (r >> 1) & 7;
    return ((x & 1) << 1) | ((x >> 1) & 1) | (x & 4);
}
template <int RB, bool FAST>
__device__ __forceinline__ int swz(int r, int c)
{
    if constexpr (FAST) {
        if constexpr (RB == 256) return swz_pi(c) ^ swz_f(r);
        else return c ^ swz_g(r);
    } else {
        if constexpr (RB == 256) return c ^ swz_x256(r);
        else return c ^ swz_x128(r);
    }
}
// the chunk stored in slot `slot` of row r
template <int RB, bool FAST>
__device__ __forceinline__ int swz_chunk(int r, int slot)
{
    if constexpr (FAST) {
        if constexpr (RB == 256) return swz_pi_inv(slot ^ swz_f(r));
        else return slot ^ swz_g(r);
    } else {
        return swz<RB, false>(r, slot);      // XOR: an involution
    }
}

// Byte offset of bf16 element (r, col) inside an RB-row tile.
template <int RB, bool FAST>
__device__ __forceinline__ int tile_off(int r, int col)
{
    return r * RB + swz<RB, FAST>(r, col >> 3) * 16 + (col & 7) * 2;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One ds_read_b64_tr_b16.  Within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte reads made by lanes 4k + i/4 of its group, k = 0..3
// (layout measured on gfx950).
__device__ __forceinline__ u32x2 lds_tr16(const char* p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Direct-to-LDS copy of `rows` rows of a bf16 [*, D] array into an RB-row tile
// (swizzled), by one wave: each instruction moves 1 KB.  `r` covers the source
// rows (rows past its end read as zeros); chunks past D are filled with zeros.
template <int D, int RB, bool FAST>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, char* tile, int row0, int rows, int lane)
{
    constexpr int SLOTS = RB / 16, ROWS_PER = 1024 / RB, CPR = D / 8;
    for (int base = row0; base < row0 + rows; base += ROWS_PER) {
        const int row = base + lane / SLOTS;
        const int c = swz_chunk<RB, FAST>(row, lane % SLOTS);
        const uint32_t off = c < CPR ? (uint32_t)(row * D * 2 + c * 16) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(tile + base * RB),
                                                 16, off, 0, 0, 0);
    }
}

// Per-lane byte offsets into RB-row swizzled tiles, computed once, so that every
// fragment read in a loop is (lane offset) + (compile-time constant).  The swizzle
// depends only on a row's low four bits, so moving by a multiple of 16 rows is a
// constant offset.
//   row(tile, m0, s): 16-byte row read, rows m0 + lane%32, chunk 2 s + lane/32
//   tr(tile, k0, jt): the MFMA operand fragment (8 bf16) for a lane that needs
//     X[k][m] with m = 32 jt + lane%32 and k = k0 + 8 (e/4) + 4 (lane/32) + e%4,
//     e = 0..7, from a row-major (k rows, m columns) tile: two transpose reads.
//     Within each group of 16 lanes, ds_read_b64_tr_b16 hands lane i element i%4
//     of the reads of lanes 4k + i/4 (k = 0..3), so lane 16g + j reads row
//     k0 + 4 (g/2) + j/4, columns 32 jt + 16 (g%2) + 4 (j%4) .. +3.
//   init(lane, row0): every offset moved down by row0 rows (row0 a multiple of 16, so the
//     swizzle is unchanged), for a wave that always reads from its own row band: the
//     wave-uniform band then costs nothing per read, instead of an address register per
//     (buffer, contraction step) pair.
template <int RB, int NKS, int NJT, bool FAST>
struct TileLane {
    int ro[NKS];
    int ta[FAST ? NJT : 2], tb[FAST ? NJT : 1];
    __device__ __forceinline__ void init(int lane, int row0 = 0)
    {
        const int l32 = lane & 31, h = lane >> 5;
        const int band = row0 * RB;
#pragma unroll
        for (int s = 0; s < NKS; ++s) ro[s] = band + l32 * RB + swz<RB, FAST>(l32, 2 * s + h) * 16;
        const int g = lane >> 4, j = lane & 15;
        const int rl = 4 * (g >> 1) + (j >> 2);            // row within the 8-row group
        const int cl = 16 * (g & 1) + 4 * (j & 3);         // column within the 32-column tile
        if constexpr (FAST) {
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                ta[jt] = band + tile_off<RB, FAST>(rl, 32 * jt + cl);
                tb[jt] = band + tile_off<RB, FAST>(rl + 8, 32 * jt + cl);
            }
        } else {
            ta[0] = band + tile_off<RB, FAST>(rl, cl);
            ta[1] = band + tile_off<RB, FAST>(rl, 32 + cl);
        }
    }
    __device__ __forceinline__ bf16x8 row(const char* tile, int m0, int s) const
    {
        return __builtin_bit_cast(bf16x8, ld16(tile + m0 * RB + ro[s]));
    }
    __device__ __forceinline__ bf16x8 tr(const char* tile, int k0, int jt) const
    {
        int o, o2;
        if constexpr (FAST) {
            o = k0 * RB + ta[jt];
            o2 = k0 * RB + tb[jt];
        } else if constexpr (RB == 256) {
            // column tile jt: slot = (4 jt) ^ T, i.e. +128 B for jt >= 2 and tile parity via ta[jt & 1];
            // row + 8 flips slot bit 3: +/-128 B
            o = k0 * RB + ((jt & 2) ? 128 : 0) + ta[jt & 1];
            o2 = o + 8 * RB + ((jt & 2) ? -128 : 128);
        } else {
            o = k0 * RB + ta[jt & 1];
            o2 = o + 8 * RB + (jt ? -64 : 64);
        }
        const u32x2 a = lds_tr16(tile + o);
        const u32x2 b = lds_tr16(tile + o2);
        return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
    }
};

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier over LDS only: this wave's LDS operations complete (lgkmcnt(0)),
// then s_barrier.  __syncthreads() releases with a fence that also waits for every
// direct-to-LDS load in flight (those write LDS); here such loads, and global stores,
// stay in flight, so the LDS they target must not be read before a wait_vmem_all()
// and a barrier.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0); vmcnt, expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) (other counters left unconstrained), n <= 63: waits until at
// most n vector-memory instructions of this wave are outstanding.
__device__ __forceinline__ void wait_vmem_leave(int n)
{
    switch (n) {   // the immediate must be a constant
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 16: __builtin_amdgcn_s_waitcnt(0x0F70 | (16 & 15) | ((16 >> 4) << 14)); break;
        case 32: __builtin_amdgcn_s_waitcnt(0x0F70 | (32 & 15) | ((32 >> 4) << 14)); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier: each call asks the
// scheduler for a group of n instructions of one class, groups issued in call order.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// max(a, b, c) in one v_max3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Lane with the same query in the other half of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest p the forward lets a probability reach before it moves its reference
// max: 2^8 (log2 units).  Keeps fp32 sums and bf16 probabilities far from overflow.
constexpr float kLazyLog2 = 8.0f;

// Sum of the two bf16 halves of x added to acc (v_dot2_f32_bf16 against ones).
__device__ __forceinline__ float sum2_bf16(uint32_t x, float acc)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), ones, acc, false);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Compute units of the current device, looked up once per device (persistent grids
// are sized by it).
inline hipError_t device_cu_count(int* n)
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    int v = (dev >= 0 && dev < 64) ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (v == 0) {
        if (hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev); e != hipSuccess)
            return e;
        if (v < 1) return hipErrorInvalidDevice;
        if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    }
    *n = v;
    return hipSuccess;
}

// Workgroup index -> logical index so that consecutive logical indices (the
// blocks of one head) run on the same XCD and share its L2.  Hardware hands
// workgroups to the 8 XCDs round-robin.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int nb) {
    if ((nb & 7) != 0) return bid;
    return (bid & 7) * (nb >> 3) + (bid >> 3);
}

// Workgroup -> (head, block).  Non-causal: the blocks of one head run back to back
// on one XCD (xcd_remap).  Causal: a block's cost grows linearly with its index.
// Each XCD works through its own heads in groups of G, a group's blocks
// longest-first (the heaviest block of every head in the group before any lighter
// one), the next group's heavy blocks filling the slots its light blocks free.
// G is the smallest head count whose blocks fill the XCD's `slots` workgroup slots,
// so the tail stays short while the K/V of only G heads compete for the XCD's L2.
// HEAVY_LAST: a head's last block costs most (query-side kernels); otherwise its
// first (key-side kernels).  Without 8 | BH the whole GPU is one group sequence.
// The query-side grids are dispatched by the hardware: an XCD hands its workgroups out
// in order, consecutive ones to its four shader engines in turn, and waits for a free
// CU in the engine whose turn it is (measured: four consecutive workgroups start
// together, once the slowest of the four before them has finished).  So there G is a
// multiple of four (or all of the XCD's heads), which makes every four consecutive
// workgroups four heads' blocks of equal cost (with whole XCD rows; without them consecutive
// workgroups go to different XCDs).  The key side walks its items itself and keeps G.
// (`slots` comes from the launch-parameter table of attn_tuning.h.)
template <bool CAUSAL, bool HEAVY_LAST>
__host__ __device__ __forceinline__ void block_coords(int bid, int nb, int nblk, int SLOTS, int& head, int& blk)
{
    if constexpr (!CAUSAL) {
        const int b = xcd_remap(bid, nb);
        head = b / nblk;
        blk = b - head * nblk;
    } else {
        const int BH = nb / nblk;
        const bool split = (BH & 7) == 0;
        const int hx = split ? BH >> 3 : BH;            // heads of this XCD (of the GPU)
        const int k = split ? bid >> 3 : bid;           // position in its sequence
        const int x = split ? (bid & 7) : 0;
        const int slots = split ? SLOTS : 8 * SLOTS;
        const int G0 = hx < (slots + nblk - 1) / nblk ? hx : (slots + nblk - 1) / nblk;
        const int G4 = (G0 + 3) & ~3;                   // G0 rounded up to whole shader-engine rounds
        const int G = HEAVY_LAST && split ? (hx < G4 ? hx : G4) : G0;
        const int g = k / (G * nblk);
        const int gh = G < hx - g * G ? G : hx - g * G; // heads in this group
        const int kk = k - g * G * nblk;
        const int rank = kk / gh;
        head = x * hx + g * G + (kk - rank * gh);
        blk = HEAVY_LAST ? nblk - 1 - rank : rank;
    }
}

// Persistent grids: a kernel launches about as many workgroups as the GPU holds at once
// and each walks a share of the nitems work items (the blocks block_coords numbers),
// so no workgroup waits to be dispatched behind another.  The items of an XCD keep
// block_coords's order (heavy causal blocks first); workgroup c of the P on an XCD takes
// positions c, 2P-1-c, 2P+c, 4P-1-c, ... of that XCD's sequence, which pairs each heavy
// item with a light one.  Without whole XCD rows (see block_coords) the GPU is one sequence.
template <bool CAUSAL>
__host__ __device__ __forceinline__ bool items_split(int nitems, int nblk)
{
    return CAUSAL ? ((nitems / nblk) & 7) == 0 : (nitems & 7) == 0;
}

struct ItemWalk {
    int xcd, pc, P, KX;
    bool split;
    __host__ __device__ __forceinline__ void init(int bid, int nwg, int nitems, bool split_)
    {
        split = split_;
        xcd = split ? (bid & 7) : 0;
        pc = split ? (bid >> 3) : bid;
        P = split ? (nwg >> 3) : nwg;
        KX = split ? (nitems >> 3) : nitems;
    }
    // the item of step t of this workgroup, or -1 once its share is done
    __host__ __device__ __forceinline__ int item(int t) const
    {
        const int pos = (t & 1) ? (t + 1) * P - 1 - pc : t * P + pc;
        if (pos >= KX) return -1;
        return split ? 8 * pos + xcd : pos;
    }
};

// Workgroups of a persistent grid: per_cu resident workgroups on every CU, at most one
// per item, whole XCD rows when the items split by XCD.
inline hipError_t persistent_grid(int nitems, int per_cu, bool split, int* nwg)
{
    int ncu = 0;
    if (hipError_t e = device_cu_count(&ncu); e != hipSuccess) return e;
    int n = ncu * per_cu;
    if (n > nitems) n = nitems;
    if (split) n &= ~7;                                 // nitems is a multiple of 8 here
    if (n < 1) n = 1;
    *nwg = n;
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Block-sparse masks.  A mask is uint8 [T][T] per head, T = ceil(N / kMaskBlock):
// entry (a, b) nonzero keeps the scores of query block a against key block b,
// zero drops them, so the kernels never load those tiles (FlashAttention-2
// review, 'sparse/hybrid' answer, section 3 (1): block-level sparse operation,
// only the important blocks are processed on chip).  kMaskBlock is a multiple
// of every kernel's tile edge (64 or 128 rows/keys, 32-row steps).
// ---------------------------------------------------------------------------
constexpr int kMaskBlock = 128;

// Walks the kept entries of one mask row (stride 1) or column (stride T) in
// increasing order.  The entries of a 64-block window sit in a wave-uniform bit
// mask (one byte load per lane and one ballot per window), so stepping to the
// next kept block is scalar work.  Every call must be made by all lanes of the
// wave, in wave-uniform control flow.
struct MaskWalk {
    const uint8_t* p;
    int stride, nb, w0;
    uint64_t win;

    __device__ __forceinline__ void load(int base, int lane)
    {
        w0 = base;
        const int b = base + lane;
        const bool kept = b < nb && p[(size_t)b * stride] != 0;
        win = __builtin_amdgcn_ballot_w64(kept);
    }
    __device__ __forceinline__ void init(const uint8_t* entries, int stride_, int nblocks, int lane)
    {
        p = entries;
        stride = stride_;
        nb = nblocks;
        load(0, lane);
    }
    // smallest kept block >= b (nb if none); b never decreases between calls
    __device__ __forceinline__ int next(int b, int lane)
    {
#pragma nounroll
        while (b < nb) {
            if (b >= w0 + 64) load(b, lane);
            const uint64_t bits = win >> (b - w0);
            if (bits != 0) return b + (int)__builtin_ctzll(bits);
            b = w0 + 64;
        }
        return nb;
    }
    // smallest unit >= u (U units per mask block) whose block is kept, or u_end
    __device__ __forceinline__ int next_unit(int u, int u_end, int U, int lane)
    {
        if (u >= u_end) return u_end;
        const int b = next(u / U, lane);
        const int v = b == u / U ? u : b * U;
        return v < u_end ? v : u_end;
    }
};

}  // namespace attn
