// Streaming a payload through 8-step FIFOs on one device: producer and
// consumer workgroups run concurrently in one cooperative launch, one pair
// per channel, each channel with its own 8-slot ring.
//
// Source (web page; cited by tag and section):
//   [NCCL14] "NCCL 专家课程 14：Simple、LL、LL128 的线格式、同步与真实性能边界"
//            (blog.cptz.space): "prerequisite mental model" (an 8-step ring;
//            the sender never overwrites a step the receiver has not
//            consumed, the receiver never consumes a step before it is
//            ready), "how LL publishes and waits for flags", "LL128's 128-byte
//            line", "LL128's warp-level ready check", "how Simple
//            synchronizes".
//
// Protocols (payload per step = step_bytes):
//   LL      16-byte lines {lo, flag, hi, flag}; each 8-byte half is written
//           in one access, so a line is ready once both flags are k + 1.
//   LL128   128-byte lines, 120 payload bytes + a 64-bit flag.  gfx950 does
//           not promise that a line written by eight lanes becomes visible
//           as a whole, so the producer makes the order explicit: all data
//           chunks of the step, then a release fence, then the flag words;
//           the consumer validates the flags with a wavefront vote and
//           re-reads the line after validation, as the page's receiver does.
//   Simple  raw payload; the producer publishes a tail step after a release
//           fence and the consumer waits for it.
// For every protocol the consumer publishes a head step (the next step it
// will consume) after each step, and the producer reuses slot k mod 8 only
// once head >= k - 7.
//
// Ring accesses use system-coherent loads and stores (sc0 sc1): producer and
// consumer may sit on different XCDs, whose L2 caches are not coherent with
// each other for these buffers.  Counters use agent-scope acquire/release
// atomics.  Every wait is bounded by max_spins and also ends as soon as any
// wait of the launch has failed (errors[0] != 0), so the launch always
// drains; its outputs are then unspecified.
#include "device.h"
#include "launch.h"

namespace ar {

constexpr int kStreamThreads = 256;
constexpr uint32_t kAbortCheck = 16;   // spins between looks at the error count

struct StreamArgs {
    const uint32_t *src;    // n fp32 payload values (as words)
    const float *local;     // n fp32 added to the received payload, or NULL
    float *out;             // n fp32
    int64_t n;
    uint8_t *fifo;          // channels x 8 slots x wire bytes
    uint64_t *head;         // per channel: next ring step the consumer needs
    uint64_t *tail;         // per channel (Simple): ring steps published
    uint32_t *errors;       // [0]: failed waits
    int64_t step_bytes;     // payload bytes per step
    int64_t wire_bytes;     // ring bytes per step
    int64_t total_steps;    // T = ceil(4n / step_bytes)
    int channels;
    uint64_t first_step;
    uint32_t max_spins;
};

__device__ __forceinline__ void store16_sys(uint8_t *p, u32x4 v)
{
    *reinterpret_cast<volatile u32x4 *>(p) = v;
}
__device__ __forceinline__ void store8_sys(uint8_t *p, u32x2 v)
{
    *reinterpret_cast<volatile u32x2 *>(p) = v;
}
__device__ __forceinline__ u32x4 load16_sys(const uint8_t *p)
{
    return *reinterpret_cast<const volatile u32x4 *>(p);
}
__device__ __forceinline__ uint64_t load_acquire(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_release(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool aborted(const uint32_t *errors)
{
    return __hip_atomic_load(errors, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Lane 0 waits until *counter >= target (bounded); the verdict reaches the
// whole workgroup through LDS.  Returns false if the launch must stop.
__device__ bool wait_counter(const uint64_t *counter, uint64_t target, const StreamArgs &a,
                             int *verdict)
{
    if (threadIdx.x == 0) {
        bool ok = load_acquire(counter) >= target;
        for (uint32_t s = 0; !ok && s < a.max_spins; ++s) {
            if (s % kAbortCheck == 0 && aborted(a.errors))
                break;
            ok = load_acquire(counter) >= target;
        }
        if (!ok)
            atomicAdd(a.errors, 1u);
        *verdict = ok ? 1 : 0;
    }
    __syncthreads();
    const bool go = *verdict != 0;
    __syncthreads();   // the verdict slot is reused by the next wait
    return go;
}

// Payload word w (zero past the end).
__device__ __forceinline__ uint32_t word_at(const StreamArgs &a, int64_t w)
{
    return w < a.n ? a.src[w] : 0u;
}

__device__ __forceinline__ void deliver(const StreamArgs &a, int64_t w, uint32_t bits)
{
    if (w < a.n) {
        const float v = __uint_as_float(bits);
        a.out[w] = a.local ? a.local[w] + v : v;
    }
}

// ---------------------------------------------------------------------------
template <int PROTO>
__device__ void produce(const StreamArgs &a, int c, int64_t s0, int64_t steps, int *verdict)
{
    uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    const int t = threadIdx.x;
    const int64_t nbytes = 4 * a.n;
    for (int64_t j = 0; j < steps; ++j) {
        const uint64_t k = a.first_step + (uint64_t)j;
        if (j >= 8 && !wait_counter(a.head + c, k - 7, a, verdict))
            return;
        uint8_t *slot = ring + (int64_t)(k % 8u) * a.wire_bytes;
        const int64_t b0 = (s0 + j) * a.step_bytes;
        const int64_t len = nbytes - b0 < a.step_bytes ? nbytes - b0 : a.step_bytes;
        const int64_t w0 = b0 / 4;
        if (PROTO == 0) {
            const uint32_t flag = (uint32_t)(k + 1);
            for (int64_t i = t; i < (len + 7) / 8; i += kStreamThreads)
                store16_sys(slot + 16 * i, u32x4{word_at(a, w0 + 2 * i), flag,
                                                 word_at(a, w0 + 2 * i + 1), flag});
        } else if (PROTO == 1) {
            const int64_t lines = (len + 119) / 120;
            for (int64_t q = t; q < lines * 8; q += kStreamThreads) {
                const int64_t l = q >> 3;
                const int ch = (int)(q & 7);
                const int64_t w = w0 + 30 * l + 4 * ch;
                if (ch < 7)
                    store16_sys(slot + 128 * l + 16 * ch,
                                u32x4{word_at(a, w), word_at(a, w + 1), word_at(a, w + 2),
                                      word_at(a, w + 3)});
                else
                    store8_sys(slot + 128 * l + 112, u32x2{word_at(a, w), word_at(a, w + 1)});
            }
            __threadfence();     // this lane's data is visible before ...
            __syncthreads();     // ... any lane of the workgroup writes a flag
            const uint64_t flag = k + 1;
            for (int64_t l = t; l < lines; l += kStreamThreads)
                store8_sys(slot + 128 * l + 120, u32x2{(uint32_t)flag, (uint32_t)(flag >> 32)});
        } else {
            const int64_t words = len / 4;
            for (int64_t q = t; q < (words + 3) / 4; q += kStreamThreads) {
                const int64_t w = w0 + 4 * q;
                if (4 * q + 3 < words)
                    store16_sys(slot + 16 * q, u32x4{word_at(a, w), word_at(a, w + 1),
                                                     word_at(a, w + 2), word_at(a, w + 3)});
                else
                    for (int64_t e = 4 * q; e < words; ++e)
                        *reinterpret_cast<volatile uint32_t *>(slot + 4 * e) = word_at(a, w0 + e);
            }
            __threadfence();
            __syncthreads();
            if (t == 0)
                store_release(a.tail + c, k + 1);
        }
    }
}

template <int PROTO>
__device__ void consume(const StreamArgs &a, int c, int64_t s0, int64_t steps, int *verdict)
{
    const uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int64_t nbytes = 4 * a.n;
    for (int64_t j = 0; j < steps; ++j) {
        const uint64_t k = a.first_step + (uint64_t)j;
        const uint8_t *slot = ring + (int64_t)(k % 8u) * a.wire_bytes;
        const int64_t b0 = (s0 + j) * a.step_bytes;
        const int64_t len = nbytes - b0 < a.step_bytes ? nbytes - b0 : a.step_bytes;
        const int64_t w0 = b0 / 4;
        bool failed = false;
        if (PROTO == 0) {
            const uint32_t flag = (uint32_t)(k + 1);
            for (int64_t i = t; i < (len + 7) / 8; i += kStreamThreads) {
                u32x4 v = load16_sys(slot + 16 * i);
                bool ok = v.y == flag && v.w == flag;
                for (uint32_t s = 0; !ok && s < a.max_spins; ++s) {
                    if (s % kAbortCheck == 0 && aborted(a.errors))
                        break;
                    v = load16_sys(slot + 16 * i);
                    ok = v.y == flag && v.w == flag;
                }
                if (!ok) {
                    failed = true;
                    break;
                }
                deliver(a, w0 + 2 * i, v.x);
                deliver(a, w0 + 2 * i + 1, v.z);
            }
        } else if (PROTO == 1) {
            const int64_t lines = (len + 119) / 120;
            const uint64_t flag = k + 1;
            const uint32_t flo = (uint32_t)flag, fhi = (uint32_t)(flag >> 32);
            // every lane runs every round (the vote is wavefront-wide)
            for (int64_t base = 0; base < lines * 8; base += kStreamThreads) {
                const int64_t q = base + t;
                const int64_t l = q >> 3;
                const int ch = (int)(q & 7);
                const bool live = l < lines;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (live)
                    v = load16_sys(slot + 128 * l + 16 * ch);
                bool ok = !live || ch != 7 || (v.z == flo && v.w == fhi);
                uint64_t mask = __ballot(!ok);
                for (uint32_t s = 0; mask != 0 && s < a.max_spins; ++s) {
                    if (s % kAbortCheck == 0 && aborted(a.errors))
                        break;
                    if (live && ((mask >> (lane | 7)) & 1u))
                        v = load16_sys(slot + 128 * l + 16 * ch);
                    ok = !live || ch != 7 || (v.z == flo && v.w == fhi);
                    mask = __ballot(!ok);
                }
                if (mask != 0) {
                    failed = true;
                    break;       // wavefront-uniform: mask is the same in every lane
                }
                // the flag is seen: re-read the chunk, now ordered after it
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if (live) {
                    v = load16_sys(slot + 128 * l + 16 * ch);
                    const int64_t w = w0 + 30 * l + 4 * ch;
                    deliver(a, w, v.x);
                    deliver(a, w + 1, v.y);
                    if (ch < 7) {
                        deliver(a, w + 2, v.z);
                        deliver(a, w + 3, v.w);
                    }
                }
            }
        } else {
            if (!wait_counter(a.tail + c, k + 1, a, verdict))
                return;
            const int64_t words = len / 4;
            for (int64_t q = t; q < (words + 3) / 4; q += kStreamThreads) {
                const u32x4 v = load16_sys(slot + 16 * q);
                for (int e = 0; e < 4; ++e)
                    if (4 * q + e < words)
                        deliver(a, w0 + 4 * q + e, v[e]);
            }
        }
        if (failed)
            atomicAdd(a.errors, 1u);
        // all lanes have their data of step k in registers: release the slot
        __syncthreads();
        if (t == 0) {
            *verdict = aborted(a.errors) ? 0 : 1;
            if (*verdict)
                store_release(a.head + c, k + 1);
        }
        __syncthreads();
        const bool go = *verdict != 0;
        __syncthreads();
        if (!go)
            return;
    }
}

// Blocks [0, channels) produce, [channels, 2 * channels) consume.
template <int PROTO>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(StreamArgs a)
{
    __shared__ int verdict;
    const int b = blockIdx.x;
    const int c = b < a.channels ? b : b - a.channels;
    const int64_t s0 = (int64_t)c * a.total_steps / a.channels;
    const int64_t s1 = (int64_t)(c + 1) * a.total_steps / a.channels;
    if (b < a.channels)
        produce<PROTO>(a, c, s0, s1 - s0, &verdict);
    else
        consume<PROTO>(a, c, s0, s1 - s0, &verdict);
}

hipError_t launch_fifo_stream(int proto, const float *src, const float *local, float *out,
                              int64_t n, void *fifo, uint64_t *counters, int channels,
                              int64_t step_bytes, int64_t wire_bytes, uint64_t first_step,
                              uint32_t max_spins, uint32_t *errors, hipStream_t s)
{
    StreamArgs a;
    a.src = reinterpret_cast<const uint32_t *>(src);
    a.local = local;
    a.out = out;
    a.n = n;
    a.fifo = static_cast<uint8_t *>(fifo);
    a.head = counters;
    a.tail = counters + channels;
    a.errors = errors;
    a.step_bytes = step_bytes;
    a.wire_bytes = wire_bytes;
    a.total_steps = (4 * n + step_bytes - 1) / step_bytes;
    a.channels = channels;
    a.first_step = first_step;
    a.max_spins = max_spins;
    void *args[] = {&a};
    const void *fn = proto == 0   ? reinterpret_cast<const void *>(&stream_kernel<0>)
                     : proto == 1 ? reinterpret_cast<const void *>(&stream_kernel<1>)
                                  : reinterpret_cast<const void *>(&stream_kernel<2>);
    return hipLaunchCooperativeKernel(fn, dim3(2 * channels), dim3(kStreamThreads), args, 0, s);
}

}  // namespace ar
