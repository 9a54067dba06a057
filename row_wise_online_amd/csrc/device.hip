// Per-device properties the plans depend on: the compute-unit count (grid
// sizes, the AUTO thresholds) and whether the device is a gfx950, the only
// architecture the kernels are built for.  Read once per device and cached;
// the first call on a device may come from several host threads at once.
#include <mutex>
#include <string.h>

#include "launch.hpp"

namespace os {
namespace {

constexpr int kMaxDevices = 64;

struct Entry {
    std::once_flag once;
    bool ok;
    Device dev;
};

Entry g_devices[kMaxDevices];

bool names_gfx950(const char *arch) {
    // gcnArchName is the target id: "gfx950", optionally followed by
    // ":feature+..." settings
    return strncmp(arch, "gfx950", 6) == 0 && (arch[6] == '\0' || arch[6] == ':');
}

}  // namespace

const Device *current_device() {
    int id = -1;
    if (hipGetDevice(&id) != hipSuccess) {
        (void)hipGetLastError();  // the failed query is ours: clear it
        return nullptr;
    }
    if (id < 0 || id >= kMaxDevices) return nullptr;
    Entry &e = g_devices[id];
    std::call_once(e.once, [&e, id] {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, id) != hipSuccess) {
            (void)hipGetLastError();
            e.ok = false;
            return;
        }
        e.dev.cus = p.multiProcessorCount;
        e.dev.gfx950 = names_gfx950(p.gcnArchName);
        e.ok = e.dev.cus > 0;
    });
    return e.ok ? &e.dev : nullptr;
}

}  // namespace os
