// Launch recorder: a host-only stand-in for the few HIP runtime entry points
// that the library's host code calls, so that its argument marshalling, its
// launch plans (kernel, grid, block, dynamic LDS, stream) and its workspace
// handling can be checked on a machine without a GPU.  Test infrastructure:
// the library's sources are compiled host-only (no device code) and linked
// against this file instead of the HIP runtime; nothing runs on a device and
// no kernel body executes.
//
// What a launch looks like from host code: kernel<<<g, b, lds, s>>>(args)
// pushes the launch configuration, then calls the kernel's host stub, which
// pops it and calls hipLaunchKernel with the stub's address and an array of
// pointers to the argument values.  The stub's address is mapped to the
// kernel's (mangled) name through the registration calls that every
// translation unit's constructor makes.
//
// Arguments are decoded only for kernels whose parameter types the test has
// declared (rec_decode): the pointer array carries no count.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

namespace {

struct Launch {
    std::string name;
    unsigned grid[3], block[3];
    size_t lds;
    void *stream;
    std::vector<uint64_t> args;
};

struct Config {
    dim3 grid, block;
    size_t lds;
    hipStream_t stream;
};

// The library's translation units register their kernels from their own
// constructors, which may run before this file's: every container is built
// on first use.
struct State {
    std::map<const void *, std::string> kernels;   // host stub -> mangled kernel name
    std::map<const void *, std::string> vars;      // host stand-in -> device variable name
    std::vector<std::pair<std::string, std::string>> decoders;   // name fragment -> parameter types
    std::vector<Launch> launches;
    int symbol_queries = 0;
    int modules = 0;
};
State &st() {
    static State s;
    return s;
}
std::mutex g_mu;   // constant-initialised
std::vector<Config> &config_stack() {
    thread_local std::vector<Config> c;
    return c;
}

// Fake device addresses handed out for device variables: far from any host
// mapping, so a host address passed where the device address belongs shows.
constexpr uint64_t kFakeDeviceBase = 0x7f5a00000000ull;

uint64_t fake_device_address(const void *host_var) {
    uint64_t i = 0;
    for (const auto &kv : st().vars) {
        if (kv.first == host_var) return kFakeDeviceBase + (i << 32);
        ++i;
    }
    return 0;
}

}  // namespace

extern "C" {

// ---- registration (each translation unit's constructor) ----
void **__hipRegisterFatBinary(const void *) {
    std::lock_guard<std::mutex> lock(g_mu);
    ++st().modules;
    static void *handle = nullptr;
    return &handle;
}
void __hipUnregisterFatBinary(void **) {}
void __hipRegisterFunction(void **, const void *hostFunction, char *, const char *deviceName, unsigned int, uint3 *,
                           uint3 *, dim3 *, dim3 *, int *) {
    std::lock_guard<std::mutex> lock(g_mu);
    st().kernels[hostFunction] = deviceName ? deviceName : "";
}
void __hipRegisterVar(void **, void *var, char *, char *deviceVar, int, size_t, int, int) {
    std::lock_guard<std::mutex> lock(g_mu);
    st().vars[var] = deviceVar ? deviceVar : "";
}

// ---- launches ----
hipError_t __hipPushCallConfiguration(dim3 gridDim, dim3 blockDim, size_t sharedMem, hipStream_t stream) {
    config_stack().push_back(Config{gridDim, blockDim, sharedMem, stream});
    return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3 *gridDim, dim3 *blockDim, size_t *sharedMem, hipStream_t *stream) {
    if (config_stack().empty()) return hipErrorInvalidConfiguration;
    const Config c = config_stack().back();
    config_stack().pop_back();
    *gridDim = c.grid;
    *blockDim = c.block;
    *sharedMem = c.lds;
    *stream = c.stream;
    return hipSuccess;
}
hipError_t hipLaunchKernel(const void *function_address, dim3 numBlocks, dim3 dimBlocks, void **args,
                           size_t sharedMemBytes, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    Launch l;
    auto it = st().kernels.find(function_address);
    l.name = it == st().kernels.end() ? std::string("?") : it->second;
    l.grid[0] = numBlocks.x; l.grid[1] = numBlocks.y; l.grid[2] = numBlocks.z;
    l.block[0] = dimBlocks.x; l.block[1] = dimBlocks.y; l.block[2] = dimBlocks.z;
    l.lds = sharedMemBytes;
    l.stream = stream;
    for (const auto &d : st().decoders) {
        if (l.name.find(d.first) == std::string::npos) continue;
        // types: p pointer, l 64-bit integer, i 32-bit integer, f float
        for (size_t a = 0; a < d.second.size(); ++a) {
            uint64_t v = 0;
            switch (d.second[a]) {
            case 'p': case 'l': std::memcpy(&v, args[a], 8); break;
            case 'i': { int32_t x; std::memcpy(&x, args[a], 4); v = (uint64_t)(int64_t)x; break; }
            case 'f': { uint32_t x; std::memcpy(&x, args[a], 4); v = x; break; }
            default: break;
            }
            l.args.push_back(v);
        }
        break;
    }
    st().launches.push_back(std::move(l));
    return hipSuccess;
}

// ---- queries ----
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "recorded launch"; }
hipError_t hipGetDevice(int *device) {
    *device = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *pi, hipDeviceAttribute_t attr, int) {
    // MI355X: 160 KB of LDS per workgroup, 256 compute units
    if (attr == hipDeviceAttributeMaxSharedMemoryPerBlock) *pi = 160 * 1024;
    else if (attr == hipDeviceAttributeMultiprocessorCount) *pi = 256;
    else return hipErrorInvalidValue;
    return hipSuccess;
}
hipError_t hipFuncGetAttributes(hipFuncAttributes *attr, const void *) {
    std::memset(attr, 0, sizeof(*attr));
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void **devPtr, const void *symbol) {
    std::lock_guard<std::mutex> lock(g_mu);
    ++st().symbol_queries;
    const uint64_t a = fake_device_address(symbol);
    if (!a) return hipErrorInvalidSymbol;
    *devPtr = reinterpret_cast<void *>(a);
    return hipSuccess;
}

// ---- the test's side ----
void rec_reset(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    st().launches.clear();
    st().decoders.clear();
}
void rec_decode(const char *name_fragment, const char *types) {
    std::lock_guard<std::mutex> lock(g_mu);
    st().decoders.emplace_back(name_fragment, types);
}
int rec_count(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    return (int)st().launches.size();
}
int rec_get(int i, char *name, int name_len, unsigned *grid3, unsigned *block3, size_t *lds, void **stream,
            uint64_t *args, int max_args) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (i < 0 || i >= (int)st().launches.size()) return -1;
    const Launch &l = st().launches[(size_t)i];
    std::strncpy(name, l.name.c_str(), (size_t)name_len - 1);
    name[name_len - 1] = 0;
    for (int d = 0; d < 3; ++d) {
        grid3[d] = l.grid[d];
        block3[d] = l.block[d];
    }
    *lds = l.lds;
    *stream = l.stream;
    const int n = (int)l.args.size() < max_args ? (int)l.args.size() : max_args;
    for (int a = 0; a < n; ++a) args[a] = l.args[(size_t)a];
    return (int)l.args.size();
}
// device address handed out for the registered device variable whose name
// contains the fragment (0 if none)
uint64_t rec_device_address(const char *name_fragment) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (const auto &kv : st().vars)
        if (kv.second.find(name_fragment) != std::string::npos) return fake_device_address(kv.first);
    return 0;
}
// host stand-in of that variable (the address the library must not pass)
uint64_t rec_host_stand_in(const char *name_fragment) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (const auto &kv : st().vars)
        if (kv.second.find(name_fragment) != std::string::npos) return (uint64_t)(uintptr_t)kv.first;
    return 0;
}
int rec_symbol_queries(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    return st().symbol_queries;
}
int rec_modules(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    return st().modules;
}

}  // extern "C"
