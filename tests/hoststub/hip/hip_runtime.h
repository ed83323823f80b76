// Host-only stand-in for the HIP runtime API used by the engine's host code.
// TEST INFRASTRUCTURE ONLY: tests/test_abi_contract.py compiles the library's
// engine.cpp with g++ against this header and hoststub.cpp, so that the
// C ABI's state machine (validation, slot states, queues, positions, columns)
// can be exercised without a GPU.  "Device" memory is host memory, streams
// run their work at once, and a captured graph is the list of launcher calls
// recorded while capturing, replayed on launch.  Never part of the product.
#pragma once
#include <stddef.h>
#include <stdint.h>

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorLaunchFailure = 719 };
typedef struct stub_stream* hipStream_t;
typedef struct stub_event* hipEvent_t;
typedef struct stub_graph* hipGraph_t;
typedef struct stub_graph_exec* hipGraphExec_t;
typedef struct stub_node* hipGraphNode_t;
enum hipMemcpyKind { hipMemcpyHostToHost = 0, hipMemcpyHostToDevice, hipMemcpyDeviceToHost, hipMemcpyDeviceToDevice,
                     hipMemcpyDefault };
enum hipStreamCaptureMode { hipStreamCaptureModeGlobal = 0, hipStreamCaptureModeThreadLocal,
                            hipStreamCaptureModeRelaxed };
enum hipFuncAttribute { hipFuncAttributeMaxDynamicSharedMemorySize = 8 };
#define hipHostMallocDefault 0u
#define hipStreamNonBlocking 1u
#define hipEventDisableTiming 2u
#define HIP_SYMBOL(x) (&(x))

const char* hipGetErrorString(hipError_t e);
hipError_t hipGetLastError();
hipError_t hipHostMalloc(void** p, size_t n, unsigned flags);
hipError_t hipHostFree(void* p);
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind k);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind k, hipStream_t s);
hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                            hipMemcpyKind k, hipStream_t s);
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t s);
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned flags);
hipError_t hipStreamDestroy(hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned flags);
hipError_t hipStreamBeginCapture(hipStream_t s, hipStreamCaptureMode m);
hipError_t hipStreamEndCapture(hipStream_t s, hipGraph_t* g);
hipError_t hipGraphInstantiate(hipGraphExec_t* e, hipGraph_t g, hipGraphNode_t* err_node, char* log, size_t n);
hipError_t hipGraphLaunch(hipGraphExec_t e, hipStream_t s);
hipError_t hipGraphExecDestroy(hipGraphExec_t e);
hipError_t hipGraphDestroy(hipGraph_t g);
hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned flags);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipGetDevice(int* d);
