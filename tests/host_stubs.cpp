// Host-only stand-ins for libsanta's kernel launchers and device-scratch
// lookup, so that the C-ABI layer (santa_api.cpp) can be built with the
// address and undefined-behaviour sanitizers on a machine without a GPU.
// Each stub reads every byte of the launch arguments it receives (so a copy
// of uninitialised or out-of-range host memory into them is caught) and
// enqueues nothing; the device-scratch lookup returns a host array that no
// stub dereferences.
#include "../sampled_sparse_decode_amd/csrc/santa_internal.h"

namespace santa {
namespace {

volatile uint64_t g_sink;
uint64_t g_launches;

template <class T>
santa_status touch(const T &x) {
    const unsigned char *b = reinterpret_cast<const unsigned char *>(&x);
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < sizeof x; ++i) h = (h ^ b[i]) * 1099511628211ull;
    g_sink = h;
    ++g_launches;
    return SANTA_OK;
}

}  // namespace

santa_status launch_build_reps(const Params &p, void *) { return touch(p); }
santa_status launch_select(const Params &p, void *) { return touch(p); }
santa_status launch_given(const Params &p, void *) { return touch(p); }
santa_status launch_gather(const Params &p, void *) { return touch(p); }
santa_status launch_combine(const Params &p, void *) { return touch(p); }
santa_status launch_value_sample(const Params &p, void *) { return touch(p); }
santa_status launch_pack_pages(const PackParams &pp, void *) { return touch(pp); }
santa_status launch_append_kv(const AppendParams &ap, void *) { return touch(ap); }
santa_status launch_pack_hashed(const ClusterParams &c, void *) { return touch(c); }
santa_status launch_pack_kmeans(const ClusterParams &c, int32_t, void *) { return touch(c); }

santa_status noalloc_scratch(void *, void **ptr) {
    alignas(256) static unsigned char host_stand_in[256];
    *ptr = host_stand_in;
    return SANTA_OK;
}

}  // namespace santa

extern "C" unsigned long long santa_stub_launches(void) { return santa::g_launches; }
