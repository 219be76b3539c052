// Optional per-kernel timing: a pair of hipEvents recorded on the launch's
// stream around each kernel the entry points enqueue.  Host code only.
#include <vector>

#include "lmoe_internal.hpp"

namespace lmoe {

namespace {
struct Recorder {
    bool on = false;
    bool open = false;
    int cap = 0;
    int n = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<const char*> names;
};
Recorder g_rec;

void release() {
    for (hipEvent_t e : g_rec.ev) (void)hipEventDestroy(e);
    g_rec = Recorder{};
}
}  // namespace

void timer_mark_begin(const char* name, hipStream_t s) {
    g_rec.open = false;
    if (!g_rec.on || g_rec.n >= g_rec.cap) return;
    if (hipEventRecord(g_rec.ev[2 * g_rec.n], s) != hipSuccess) return;
    g_rec.names[g_rec.n] = name;
    g_rec.open = true;
}

void timer_mark_end(hipStream_t s) {
    if (!g_rec.open) return;
    g_rec.open = false;
    if (hipEventRecord(g_rec.ev[2 * g_rec.n + 1], s) == hipSuccess) ++g_rec.n;
}

}  // namespace lmoe

using namespace lmoe;

extern "C" {

int lmoe_timing_start(int capacity) {
    release();
    if (capacity < 1 || capacity > (1 << 20)) return LMOE_ERR_SHAPE;
    g_rec.ev.reserve(2 * (size_t)capacity);
    for (int i = 0; i < 2 * capacity; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            release();
            return LMOE_ERR_HIP;
        }
        g_rec.ev.push_back(e);
    }
    g_rec.names.assign(capacity, nullptr);
    g_rec.cap = capacity;
    g_rec.on = true;
    return LMOE_OK;
}

int lmoe_timing_stop(lmoe_kernel_time* out, int capacity, int* count) {
    int st = LMOE_OK;
    int written = 0;
    for (int i = 0; i < g_rec.n; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_rec.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_rec.ev[2 * i], g_rec.ev[2 * i + 1]) != hipSuccess) {
            st = LMOE_ERR_HIP;
            break;
        }
        if (out && written < capacity) out[written++] = lmoe_kernel_time{g_rec.names[i], ms};
    }
    if (count) *count = written;
    release();
    return st;
}

}  // extern "C"
