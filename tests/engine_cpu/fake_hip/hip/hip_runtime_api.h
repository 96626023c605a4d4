// A host-only stand-in for the HIP runtime API, used to build the sliding
// engine's host logic (engine.cpp, adam.cpp, layout.cpp) on the CPU for the
// race and ordering checks in tests/engine_cpu.  It declares only what those
// files use; fake_hip.cpp implements it with one worker thread per stream
// and events with the runtime's ordering rules.  Test infrastructure: the
// library never includes it.
#pragma once

#include <cstddef>
#include <cstdint>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNotReady = 600,
  hipErrorUnknown = 999,
} hipError_t;

struct FakeStream;
struct FakeEvent;
typedef FakeStream* hipStream_t;
typedef FakeEvent* hipEvent_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4,
} hipMemcpyKind;

typedef enum hipMemoryType {
  hipMemoryTypeUnregistered = 0,
  hipMemoryTypeHost = 1,
  hipMemoryTypeDevice = 2,
} hipMemoryType;

typedef struct hipPointerAttribute_t {
  hipMemoryType type;
  int device;
  void* devicePointer;
  void* hostPointer;
} hipPointerAttribute_t;

#define hipStreamDefault 0x0
#define hipStreamNonBlocking 0x1
#define hipEventDefault 0x0
#define hipEventDisableTiming 0x2
#define hipHostMallocDefault 0x0

hipError_t hipSetDevice(int device);
hipError_t hipGetDevice(int* device);
const char* hipGetErrorString(hipError_t e);
hipError_t hipGetLastError(void);

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int flags);
hipError_t hipStreamDestroy(hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int flags);

hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned int flags);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventQuery(hipEvent_t e);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t start, hipEvent_t stop);

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t s);
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned int flags);
hipError_t hipHostFree(void* p);
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* p);
