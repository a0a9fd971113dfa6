// fp8gemm_jit.cpp -- run-time specialisation of the tiled kernel (host code).
//
// The pages' library compiles every kernel at run time, so the shape of a call is known when the
// kernel is built (page "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", section
// 深入了解DeepGEMM: no install-time compilation, a light JIT module; section 如何使用？: block
// sizes and pipeline stages chosen at JIT time).  Here the launch shape still comes from the
// ahead-of-time table; what the run-time build adds is N and K as compile-time constants of the
// same kernel body (fp8gemm_tiled.h), compiled with hipRTC for gfx950, loaded as a module and
// cached per device and (table entry, N, K) for the life of the process.
//
// The kernel sources are compiled into the library as text (fp8gemm_jit_sources.inc, generated
// by the build from fp8gemm_args.h, fp8gemm_device.h and fp8gemm_tiled.h); the two system headers
// they include are replaced by the stand-ins below, since hipRTC provides the HIP device
// built-ins itself.
//
// hipRTC is loaded at first use into a linker namespace of its own (dlmopen), from
// $FP8GEMM_HIPRTC, else $ROCM_PATH/lib/libhiprtc.so.7, else /opt/rocm/lib/libhiprtc.so.7.  A
// process may already hold another ROCm's hipRTC and code-object compiler under the same names
// (PyTorch wheels bundle their own); in its own namespace the library gets the ROCm compiler it
// was built with, and its code-generation options are the ahead-of-time build's.
//
// That namespace has its own C library, whose environment pointer is the process's array as it
// was at load time.  The compiler reads the environment on every compile, and setenv (Python's
// os.environ, among others) frees that array when it grows the environment, so before each
// compile the namespace's pointer is set to the process's current array, under a lock that
// serialises the compiles.  As for getenv anywhere, a setenv on another thread while a compile
// runs is the caller's race.

#include <dlfcn.h>
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <link.h>

#include <chrono>
#include <cstdlib>
#include <cstdio>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include <unistd.h>

#include "fp8gemm.h"
#include "fp8gemm_internal.h"
#include "fp8gemm_jit_sources.inc"

namespace fp8gemm {

namespace {

const char kStubHipRuntime[] = "#pragma once\n";
const char kStubStdint[] =
    "#pragma once\n"
    "typedef __UINT8_TYPE__ uint8_t;\ntypedef __UINT16_TYPE__ uint16_t;\n"
    "typedef __UINT32_TYPE__ uint32_t;\ntypedef __UINT64_TYPE__ uint64_t;\n"
    "typedef __INT8_TYPE__ int8_t;\ntypedef __INT16_TYPE__ int16_t;\n"
    "typedef __INT32_TYPE__ int32_t;\ntypedef __INT64_TYPE__ int64_t;\n"
    "typedef __UINTPTR_TYPE__ uintptr_t;\n";

// The same device code generation options as the ahead-of-time build.
const char* const kOptions[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-mllvm", "-amdgpu-mfma-vgpr-form",
                                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};

std::string name_expression(const KernelEntry& e, int N, int K) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "fp8gemm::fp8gemm_kernel<%d, %d, %d, %d, %d, %d, %d, %d>", e.bm, e.bn,
                  e.waves_m, e.waves_n, e.stages, e.layout, N, K);
    return buf;
}

// The hipRTC entry points, resolved in the library's own namespace.
struct Rtc {
    decltype(&hiprtcCreateProgram) create = nullptr;
    decltype(&hiprtcDestroyProgram) destroy = nullptr;
    decltype(&hiprtcAddNameExpression) add_name = nullptr;
    decltype(&hiprtcCompileProgram) compile = nullptr;
    decltype(&hiprtcGetProgramLogSize) log_size = nullptr;
    decltype(&hiprtcGetProgramLog) log = nullptr;
    decltype(&hiprtcGetLoweredName) lowered = nullptr;
    decltype(&hiprtcGetCodeSize) code_size = nullptr;
    decltype(&hiprtcGetCode) code = nullptr;
    char*** environ_slot = nullptr;     // `environ` of the namespace's C library
    std::string error;
};

const Rtc& rtc() {
    static const Rtc r = [] {
        Rtc t;
        std::string path;
        if (const char* e = std::getenv("FP8GEMM_HIPRTC")) path = e;
        else if (const char* e2 = std::getenv("ROCM_PATH")) path = std::string(e2) + "/lib/libhiprtc.so.7";
        else path = "/opt/rocm/lib/libhiprtc.so.7";
        void* h = dlmopen(LM_ID_NEWLM, path.c_str(), RTLD_NOW | RTLD_LOCAL);
        if (!h) {
            const char* msg = dlerror();
            t.error = "cannot load " + path + ": " + (msg ? msg : "unknown error");
            return t;
        }
        bool ok = true;
        auto sym = [&](auto& f, const char* name) {
            f = reinterpret_cast<std::remove_reference_t<decltype(f)>>(dlsym(h, name));
            ok = ok && f != nullptr;
        };
        sym(t.create, "hiprtcCreateProgram");
        sym(t.destroy, "hiprtcDestroyProgram");
        sym(t.add_name, "hiprtcAddNameExpression");
        sym(t.compile, "hiprtcCompileProgram");
        sym(t.log_size, "hiprtcGetProgramLogSize");
        sym(t.log, "hiprtcGetProgramLog");
        sym(t.lowered, "hiprtcGetLoweredName");
        sym(t.code_size, "hiprtcGetCodeSize");
        sym(t.code, "hiprtcGetCode");
        if (!ok) {
            t = Rtc{};
            t.error = path + " lacks a hipRTC entry point";
            return t;
        }
        Lmid_t ns = 0;
        void* c = dlinfo(h, RTLD_DI_LMID, &ns) == 0 ? dlmopen(ns, "libc.so.6", RTLD_NOW | RTLD_NOLOAD) : nullptr;
        t.environ_slot = c ? reinterpret_cast<char***>(dlsym(c, "environ")) : nullptr;
        if (!t.environ_slot) {
            t = Rtc{};
            t.error = "cannot find the C library of the namespace of " + path;
        }
        return t;
    }();
    return r;
}

struct Program {
    hiprtcProgram p = nullptr;
    ~Program() {
        if (p) rtc().destroy(&p);
    }
};

struct Cached {
    hipModule_t module = nullptr;
    JitKernel k;
};

std::mutex g_mu;
std::mutex g_compile_mu;    // one compile at a time: the namespace's environment pointer is shared
std::map<std::tuple<int, int, int, int>, std::unique_ptr<Cached>> g_cache;   // (device, entry, N, K)

}  // namespace

int jit_compile(const KernelEntry& e, int N, int K, std::vector<char>* code, std::string* lowered,
                std::string* log) {
    if (e.kind != kKindTiled || N <= 0 || K <= 0 || K % 128 != 0) return FP8GEMM_ERR_BAD_SHAPE;
    const Rtc& r = rtc();
    if (!r.create) {
        if (log) *log = r.error;
        return FP8GEMM_ERR_HIP;
    }
    std::vector<const char*> headers = {kStubHipRuntime, kStubStdint};
    std::vector<const char*> names = {"hip/hip_runtime.h", "stdint.h"};
    for (int i = 0; i < kJitSourceCount; ++i) {
        headers.push_back(kJitSources[i]);
        names.push_back(kJitSourceNames[i]);
    }
    const char* src = "#include \"fp8gemm_tiled.h\"\n";
    std::lock_guard<std::mutex> lock(g_compile_mu);
    *r.environ_slot = environ;          // the process's environment as it is now
    Program prog;
    if (r.create(&prog.p, src, "fp8gemm_specialized.hip", (int)headers.size(), headers.data(),
                            names.data()) != HIPRTC_SUCCESS)
        return FP8GEMM_ERR_HIP;
    const std::string expr = name_expression(e, N, K);
    if (r.add_name(prog.p, expr.c_str()) != HIPRTC_SUCCESS) return FP8GEMM_ERR_HIP;
    const hiprtcResult cr = r.compile(prog.p, (int)(sizeof kOptions / sizeof kOptions[0]), kOptions);
    size_t log_size = 0;
    if (log && r.log_size(prog.p, &log_size) == HIPRTC_SUCCESS && log_size > 1) {
        log->assign(log_size, '\0');
        r.log(prog.p, &(*log)[0]);
    }
    if (cr != HIPRTC_SUCCESS) return FP8GEMM_ERR_HIP;
    const char* low = nullptr;
    if (r.lowered(prog.p, expr.c_str(), &low) != HIPRTC_SUCCESS || !low) return FP8GEMM_ERR_HIP;
    if (lowered) *lowered = low;
    size_t size = 0;
    if (r.code_size(prog.p, &size) != HIPRTC_SUCCESS || size == 0) return FP8GEMM_ERR_HIP;
    code->resize(size);
    if (r.code(prog.p, code->data()) != HIPRTC_SUCCESS) return FP8GEMM_ERR_HIP;
    return FP8GEMM_OK;
}

int jit_kernel(int device, const KernelEntry& e, int entry, int N, int K, const JitKernel** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_tuple(device, entry, N, K);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) {
        *out = &it->second->k;
        return FP8GEMM_OK;
    }
    const auto t0 = std::chrono::steady_clock::now();
    std::vector<char> code;
    std::string lowered, log;
    int st = jit_compile(e, N, K, &code, &lowered, &log);
    if (st != FP8GEMM_OK) {
        if (!log.empty()) std::fprintf(stderr, "[fp8gemm] run-time compile failed:\n%s\n", log.c_str());
        return st;
    }
    auto c = std::make_unique<Cached>();
    if (hipModuleLoadData(&c->module, code.data()) != hipSuccess) return FP8GEMM_ERR_HIP;
    if (hipModuleGetFunction(&c->k.fn, c->module, lowered.c_str()) != hipSuccess) {
        (void)hipModuleUnload(c->module);
        return FP8GEMM_ERR_HIP;
    }
    int blocks = 0;
    if (hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, c->k.fn, e.threads, 0) != hipSuccess ||
        blocks <= 0)
        blocks = 1;
    c->k.occupancy = blocks;
    c->k.compile_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    *out = &c->k;
    g_cache.emplace(key, std::move(c));
    return FP8GEMM_OK;
}

int jit_cache_size() {
    std::lock_guard<std::mutex> lock(g_mu);
    return (int)g_cache.size();
}

}  // namespace fp8gemm
