// synth.hip -- GPU side of the seeded synthetic input generator (untimed).
//
// Implements the same definition as bit_exact_xor_amd/synth.py, element for
// element: the i-th output of a SplitMix64 sequence (Steele, Lea, Flood,
// "Fast splittable pseudorandom number generators", OOPSLA 2014) keyed per
// generated region, turned into BF16 N(0, 0.02) weights (Irwin-Hall sum of
// four 16-bit lanes, one fp32 multiply, round-to-nearest-even to BF16), uint8
// codes or fp32 scales, and the changed element of a new version.  Holds
// nothing of the delta method itself.  Built into its own library,
// libdcr_synth.so.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t hash_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGamma); }

__device__ __forceinline__ uint16_t bf16_old(uint64_t key_old, uint64_t i, uint32_t scale_bits) {
    const uint64_t h = hash_at(key_old, i);
    const int32_t s = int32_t((h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48));
    const float x = float(s - 131070) * __uint_as_float(scale_bits);   // exact convert, one rounded multiply
    const uint32_t b = __float_as_uint(x);
    return uint16_t((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t bf16_step(uint16_t old, bool up) {
    const uint32_t o = old, mag = o & 0x7FFFu;
    if (mag == 0) return uint16_t(o | 1u);
    return uint16_t((up && mag < 0x7F7Fu) ? o + 1u : o - 1u);
}

struct Region {
    uint64_t elem_off;   // first element in the shard
    uint64_t n;          // elements
    uint64_t key_old, key_chg;
    uint64_t thr;        // change iff low 32 bits of the change hash < thr
    uint64_t row_len;    // GEN_BF16_HOT: elements per row
    uint64_t hot_off;    // GEN_BF16_HOT: first index into the hot-row list
    uint64_t key_blk;    // GEN_BF16_HOT: change key of the coupled scale region
    uint64_t thr_blk;
    uint32_t blk;        // elements per coupled block (0: none)
    uint32_t kind;       // 0 BF16, 1 U8, 2 F32 scale, 3 BF16 with hot rows / coupled blocks
    uint32_t n_hot;      // GEN_BF16_HOT: hot rows (sorted)
};

__device__ __forceinline__ bool is_hot(const uint32_t* hot, uint32_t n, uint64_t row) {
    uint32_t lo = 0, hi = n;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (hot[mid] < row) lo = mid + 1;
        else hi = mid;
    }
    return lo < n && hot[lo] == row;
}

// One thread per element of one region; version 0 = old, 1 = new.
__global__ void gen_kernel(uint8_t* shard, Region r, const uint32_t* hot, uint32_t version, uint32_t scale_bits) {
    const uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x;
    if (i >= r.n) return;
    const uint64_t e = r.elem_off + i;
    if (r.kind == 0 || r.kind == 3) {
        const uint16_t old = bf16_old(r.key_old, i, scale_bits);
        uint16_t v = old;
        if (version) {
            const uint64_t h = hash_at(r.key_chg, i);
            bool changed = (h & 0xFFFFFFFFull) < r.thr;
            if (r.kind == 3 && r.n_hot) changed = changed || is_hot(hot + r.hot_off, r.n_hot, i / r.row_len);
            if (r.kind == 3 && r.blk) changed = changed || (hash_at(r.key_blk, i / r.blk) & 0xFFFFFFFFull) < r.thr_blk;
            if (changed) v = bf16_step(old, ((h >> 32) & 1u) != 0);
        }
        reinterpret_cast<uint16_t*>(shard)[e] = v;
    } else if (r.kind == 1) {
        const uint8_t old = uint8_t(hash_at(r.key_old, i) & 0xFF);
        uint8_t v = old;
        if (version) {
            const uint64_t h = hash_at(r.key_chg, i);
            if ((h & 0xFFFFFFFFull) < r.thr) {
                const uint32_t sh = uint32_t((h >> 33) & 1u) * 4u;
                const uint32_t nib = (old >> sh) & 0xFu;
                const uint32_t nn = (nib + 1u + uint32_t((h >> 34) % 15u)) & 0xFu;
                v = uint8_t((old & ~(0xFu << sh)) | (nn << sh));
            }
        }
        shard[e] = v;
    } else {
        const uint32_t old = 0x3B000000u + uint32_t(hash_at(r.key_old, i) & 0x00FFFFFFull);
        uint32_t v = old;
        if (version) {
            const uint64_t h = hash_at(r.key_chg, i);
            if ((h & 0xFFFFFFFFull) < r.thr) v = old ^ (1u + uint32_t((h >> 40) & 0x3FFu));
        }
        reinterpret_cast<uint32_t*>(shard)[e] = v;
    }
}

// Streaming-read probe, used only to measure this GPU's read ceiling: each
// 256-thread workgroup reads one contiguous 64 KiB block with 16 non-temporal
// 128-bit loads per thread, all in flight at once, and XORs them together.
// Nothing is stored unless the fold hits one fixed value, which keeps the
// loads alive.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_probe_kernel(const v4u* buf, uint64_t n16, uint32_t* sink) {
    const uint64_t base = uint64_t(blockIdx.x) * 4096u + threadIdx.x;
    v4u x = {0, 0, 0, 0};
    if (base + 15u * 256u < n16) {
#pragma unroll
        for (uint32_t k = 0; k < 16; k++) x ^= __builtin_nontemporal_load(buf + base + k * 256u);
    } else {
        for (uint32_t k = 0; k < 16; k++)
            if (base + k * 256u < n16) x ^= __builtin_nontemporal_load(buf + base + k * 256u);
    }
    const uint32_t f = x.x ^ x.y ^ x.z ^ x.w;
    if (f == 0x9E3779B9u) sink[0] = f;
}

// Read-modify-write probe, used only to measure this GPU's ceiling for the
// access pattern of an in-place patch: every 16-byte group whose bit is set
// in `bits` (LSB first, one bit per group) is read, XORed with a fixed
// nonzero mask and written back, nothing else is touched.  Thread t owns the
// 16 consecutive groups 16t .. 16t + 15 (bits[t]).  Two runs restore the
// buffer.
__global__ __launch_bounds__(256) void rmw_probe_kernel(v4u* buf, const uint16_t* bits, uint64_t n16) {
    const uint64_t t = uint64_t(blockIdx.x) * 256u + threadIdx.x;
    const uint64_t g0 = t * 16u;
    if (g0 >= n16) return;
    uint32_t b = bits[t];
    if (n16 - g0 < 16u) b &= (1u << uint32_t(n16 - g0)) - 1u;
    const v4u m = {0x00010001u, 0x00800080u, 0x01000100u, 0x80008000u};
    while (b) {
        const uint32_t i = uint32_t(__ffs(b) - 1);
        b &= b - 1u;
        buf[g0 + i] ^= m;
    }
}

// The same patch with every touched 128-byte line read and written whole
// (eight 16-byte groups a line, counted from the buffer's start: a 128-byte
// aligned buffer gives the GPU's own lines), the access pattern of an apply
// that writes whole lines: one thread per group, the line's eight bits read
// as one byte; a grid-stride loop over the groups.
__global__ __launch_bounds__(256) void rmw_lines_probe_kernel(v4u* buf, const uint8_t* bits, uint64_t n16) {
    const uint64_t stride = uint64_t(gridDim.x) * 256u;
    const v4u m = {0x00010001u, 0x00800080u, 0x01000100u, 0x80008000u};
    for (uint64_t g = uint64_t(blockIdx.x) * 256u + threadIdx.x; g < n16; g += stride) {
        uint32_t lb = bits[g >> 3];
        const uint64_t l0 = g & ~uint64_t(7);
        if (n16 - l0 < 8u) lb &= (1u << uint32_t(n16 - l0)) - 1u;
        if (!lb) continue;
        v4u v = buf[g];
        if ((lb >> uint32_t(g & 7u)) & 1u) v ^= m;
        buf[g] = v;
    }
}

}  // namespace

extern "C" {

// Fill elements [elem_off, elem_off + n) of `shard` (device memory) with one
// generated region.  `hot` is a device array of sorted hot-row indices (or
// NULL).  Returns 0 or a HIP error code.
int32_t dcr_synth_fill(void* shard, uint64_t elem_off, uint64_t n, uint32_t kind, uint64_t key_old,
                       uint64_t key_chg, uint64_t thr, uint64_t row_len, const uint32_t* hot, uint64_t hot_off,
                       uint32_t n_hot, uint64_t key_blk, uint64_t thr_blk, uint32_t blk, uint32_t version,
                       uint32_t scale_bits, void* stream) {
    if (n == 0) return 0;
    Region r{elem_off, n, key_old, key_chg, thr, row_len ? row_len : 1, hot_off, key_blk, thr_blk, blk, kind, n_hot};
    const uint64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return int32_t(hipErrorInvalidValue);
    hipLaunchKernelGGL(gen_kernel, dim3(uint32_t(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(shard), r, hot, version, scale_bits);
    return int32_t(hipGetLastError());
}

// Read `bytes` of device memory at `buf` once (both 16-byte aligned/multiple)
// with the streaming-read probe; `sink` is 4 bytes of device memory.  Returns
// 0 or a HIP error code.
int32_t dcr_synth_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes & 15u) || !sink) return int32_t(hipErrorInvalidValue);
    if (bytes == 0) return 0;
    const uint64_t blocks = (bytes / 16 + 4095) / 4096;
    if (blocks > 0x7FFFFFFFull) return int32_t(hipErrorInvalidValue);
    hipLaunchKernelGGL(read_probe_kernel, dim3(uint32_t(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u*>(buf), bytes / 16, sink);
    return int32_t(hipGetLastError());
}

// XOR a fixed mask into every 16-byte group of `buf` (`bytes`, 16-byte
// aligned and a multiple of 16) whose bit is set in the device bit array
// `bits` (ceil(groups / 16) 16-bit words, LSB first), with the
// read-modify-write probe.  Returns 0 or a HIP error code.
int32_t dcr_synth_rmw_probe(void* buf, uint64_t bytes, const void* bits, void* stream) {
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes & 15u) || (reinterpret_cast<uintptr_t>(bits) & 1u) || !bits)
        return int32_t(hipErrorInvalidValue);
    if (bytes == 0) return 0;
    const uint64_t n16 = bytes / 16, threads = (n16 + 15) / 16, blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return int32_t(hipErrorInvalidValue);
    hipLaunchKernelGGL(rmw_probe_kernel, dim3(uint32_t(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<v4u*>(buf), static_cast<const uint16_t*>(bits), n16);
    return int32_t(hipGetLastError());
}

// The same groups patched with each touched 128-byte line (eight groups from
// the buffer's start) read and written whole.  Same arguments and checks.
int32_t dcr_synth_rmw_lines_probe(void* buf, uint64_t bytes, const void* bits, void* stream) {
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes & 15u) || (reinterpret_cast<uintptr_t>(bits) & 1u) || !bits)
        return int32_t(hipErrorInvalidValue);
    if (bytes == 0) return 0;
    const uint64_t n16 = bytes / 16, blocks = std::min<uint64_t>((n16 + 255) / 256, uint64_t(1) << 20);
    hipLaunchKernelGGL(rmw_lines_probe_kernel, dim3(uint32_t(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<v4u*>(buf), static_cast<const uint8_t*>(bits),
                       n16);
    return int32_t(hipGetLastError());
}

}  // extern "C"
