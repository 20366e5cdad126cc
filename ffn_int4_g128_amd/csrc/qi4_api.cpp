// libqi4 entry points that do not launch kernels: version, status strings,
// packed size, and the cached per-device architecture check.
#include <atomic>
#include <cstring>

#include "qi4_dev.h"
#include "qi4_host.h"

namespace qi4 {

namespace {
constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];
}  // namespace

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QI4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return QI4_ERR_UNSUPPORTED;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QI4_ERR_HIP;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? QI4_OK : QI4_ERR_UNSUPPORTED;
}

}  // namespace qi4

extern "C" {

int qi4_abi_version(void) { return QI4_ABI_VERSION; }

const char *qi4_status_string(int status) {
    switch (status) {
        case QI4_OK: return "ok";
        case QI4_ERR_NULL: return "a required pointer is NULL";
        case QI4_ERR_SHAPE: return "a size is out of range, K is not a multiple of 128, or a pointer is misaligned";
        case QI4_ERR_DTYPE: return "unknown dtype or epilogue";
        case QI4_ERR_GROUP: return "group_size must be 0, 64 or a multiple of 128";
        case QI4_ERR_WORKSPACE: return "workspace too small";
        case QI4_ERR_ALIAS: return "an output overlaps an input";
        case QI4_ERR_UNSUPPORTED: return "unsupported device (needs gfx950) or flag combination";
        case QI4_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        default: return "unknown status";
    }
}

int64_t qi4_packed_bytes(int64_t N, int64_t K, int group_size, int flags) {
    int rc = qi4::check_matrix(N, K, group_size, flags);
    if (rc != QI4_OK) return rc;
    return qi4::PackedLayout(N, qi4::packed_k(K, flags), flags,
                             (int)qi4::effective_group(group_size, K)).bytes;
}

}  // extern "C"
